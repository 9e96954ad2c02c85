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
// Work split. A workgroup of 8 waves owns 256 query tokens of one (batch, head);
// each wave owns 32 tokens and keeps their Qhat rows in registers. The waves
// walk the key window in tiles of 64 keys. A tile [64][224] is staged once in
// LDS (row-major, double-buffered) and read by all 8 waves, i.e. all query
// tokens of the block share each cache read.
//
// Per tile and wave (transposed formulation, keys on MFMA rows):
//   S^T[key][q]  = K[key][:] . Qhat[q][:]     2 key blocks x 14 MFMA 32x32x16
//   online softmax per query (= per lane): max / sum over the lane's own keys,
//   the other half of the keys sits in lane l^32 (one permlane32 swap)
//   O^T[d][q]   += C^T[d][key] . P^T[key][q]  6 latent blocks x 4 MFMA; C^T is
//   read straight from the row-major tile with the LDS transpose read, and P^T
//   is the S^T accumulator converted to bf16 in place (the MFMA contraction
//   order of keys is permuted identically on both operands).
// Epilogue: out^T[e][q] = W_V_up[h]^T[e][:] . (O^T / l)[:][q], W_V_up[h]
// staged in LDS and read transposed.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace vmla {
namespace {

constexpr int kKT = 64;                     // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockQ = 32 * kWaves;        // query tokens per workgroup
constexpr int kKLd = kRow + 8;              // padded LDS key row (elements)
constexpr int kTileElems = kKT * kKLd;
constexpr int kChunks = kKT * kRow / 8;     // 16-byte chunks per tile
constexpr int kCpt = (kChunks + kThreads - 1) / kThreads;
constexpr int kVLd = kDV + 8;               // padded LDS row of W_V_up[h]
constexpr int kFeatSteps = kRow / 16;       // 14
constexpr int kLatTiles = kDC / 32;         // 6
constexpr float kLazy = 8.f;                // lazy-rescale threshold (log2 units)
static_assert(kDC * kVLd <= 2 * kTileElems, "W_V_up staging must fit in the tile buffers");

template <typename T>
__global__ __launch_bounds__(kThreads)
void latent_attn_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t kt[2 * kTileElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int half = lane >> 5;
  const int qi = lane & 31;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int qrow = blockIdx.x * kBlockQ + 32 * wave + qi;
  const bool qvalid = qrow < a.n_q;

  // Qhat fragments (B operand of S^T): lane holds features ks*16 + 8*half + e of its query.
  const bf16_t* qp = a.qhat + (((size_t)b * a.n_heads + h) * a.n_q + (qvalid ? qrow : a.n_q - 1)) * kRow;
  bf16x8 qf[kFeatSteps];
#pragma unroll
  for (int ks = 0; ks < kFeatSteps; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(qp + ks * 16 + 8 * half);

  const T* cache = static_cast<const T*>(a.cache) + (size_t)b * a.cache_rows * kRow;
  const int ntiles = (a.n_k + kKT - 1) / kKT;

  uint4 pre[kCpt];
  auto load_tile = [&](int j) {
#pragma unroll
    for (int i = 0; i < kCpt; ++i) {
      const int c = tid + i * kThreads;
      const int key = c / (kRow / 8), cc = c % (kRow / 8);
      const int kg = j * kKT + key;
      pre[i] = make_uint4(0, 0, 0, 0);
      if (c < kChunks && kg < a.n_k) pre[i] = load8_bf16<T>(cache + (size_t)kg * kRow + 8 * cc);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kCpt; ++i) {
      const int c = tid + i * kThreads;
      const int key = c / (kRow / 8), cc = c % (kRow / 8);
      if (c < kChunks) *reinterpret_cast<uint4*>(&kt[buf * kTileElems + key * kKLd + 8 * cc]) = pre[i];
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  f32x16 o[kLatTiles];
#pragma unroll
  for (int t = 0; t < kLatTiles; ++t) o[t] = f32x16{};
  // m: reference max of this query (log2 units), identical in lanes l and l^32;
  // l: running sum over this lane's half of the keys, relative to m.
  float m = -INFINITY;
  float l = 0.f;

  // One 64-key tile. Register r of s0 / s1 holds key 8(r/4) + 4*half + r%4 of
  // the tile's first / second 32-key block.
  auto tile = [&](const bf16_t* K, int key0, auto masked) {
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kFeatSteps; ++ks) {
      const bf16x8 a0 = lds_row8(&K[qi * kKLd + ks * 16 + 8 * half]);
      const bf16x8 a1 = lds_row8(&K[(32 + qi) * kKLd + ks * 16 + 8 * half]);
      s0 = mfma32(a0, qf[ks], s0);
      s1 = mfma32(a1, qf[ks], s1);
    }
    if constexpr (decltype(masked)::value) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = key0 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (key >= a.n_k) s0[r] = -INFINITY;
        if (key + 32 >= a.n_k) s1[r] = -INFINITY;
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
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const f32x16& sv = kb ? s1 : s0;
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = (__bf16)sv[8 * jj + e];
        const int kbase = kb * 32 + jj * 16;
#pragma unroll
        for (int t = 0; t < kLatTiles; ++t) {
          const bf16x8 av = lds_tr8(K, kKLd, kbase + 4 * half, kbase + 8 + 4 * half, 32 * t, lane);
          o[t] = mfma32(av, pb, o[t]);
        }
      }
    }
  };

  // Full tiles, then the partial tail tile (if any) with key masking.
  const int nfull = a.n_k / kKT;
  for (int j = 0; j < nfull; ++j) {
    const int buf = j & 1;
    if (j + 1 < ntiles) load_tile(j + 1);
    tile(kt + buf * kTileElems, j * kKT, std::false_type{});
    if (j + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }
  if (nfull < ntiles) {
    tile(kt + (nfull & 1) * kTileElems, nfull * kKT, std::true_type{});
    __syncthreads();
  }

  // ---- epilogue: out = (O / l) @ W_V_up[h]
  const float inv = 1.f / sum_across_halves(l);
  bf16_t* wv = kt;   // [kDC][kVLd]
  const T* wsrc = static_cast<const T*>(a.w_v_up) + (size_t)h * kDC * kDV;
#pragma unroll
  for (int i = 0; i < kDC * kDV / 8 / kThreads; ++i) {
    const int c = tid + i * kThreads;
    const int row = c / (kDV / 8), cc = c % (kDV / 8);
    *reinterpret_cast<uint4*>(&wv[row * kVLd + 8 * cc]) = load8_bf16<T>(wsrc + (size_t)row * kDV + 8 * cc);
  }
  __syncthreads();

  bf16x8 ob[kLatTiles][2];
#pragma unroll
  for (int t = 0; t < kLatTiles; ++t)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int e = 0; e < 8; ++e) ob[t][jj][e] = (__bf16)(o[t][8 * jj + e] * inv);

  T* out = static_cast<T*>(a.out) + (((size_t)b * a.n_q + (qvalid ? qrow : 0)) * a.n_heads + h) * kDV;
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

}  // namespace

hipError_t launch_latent_attn(const AttnArgs& a, bool f32, hipStream_t s) {
  dim3 grid((a.n_q + kBlockQ - 1) / kBlockQ, a.n_heads, a.batch);
  if (f32) hipLaunchKernelGGL(latent_attn_kernel<float>, grid, dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(latent_attn_kernel<bf16_t>, grid, dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace vmla
