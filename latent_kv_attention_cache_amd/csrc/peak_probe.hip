// Peak probes: the measured second reference lines of the two rooflines.
//  - Matrix cores: every SIMD runs waves that issue independent back-to-back
//    v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic
//    inside the loop, so the launch time gives the sustained dense bf16 MFMA
//    rate of the chip at the clock it holds under that load.
//  - HBM: a grid-stride stream of 16-byte non-temporal loads over a buffer far
//    larger than the caches, eight loads in flight per lane, XOR-reduced so
//    they stay live: the sustained read bandwidth.
// Not part of the library's C ABI: built into its own libvmla_probe.so and
// used by bench.py only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeBlocks = 1024;    // 4 blocks of 4 waves per CU on 256 CUs: 4 waves per SIMD
constexpr int kProbeThreads = 256;
constexpr int kChains = 4;            // independent accumulators per wave, hides the MFMA latency

__global__ __launch_bounds__(kProbeThreads) void mfma_peak_kernel(float* sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(1e-3f * (float)(threadIdx.x + e));
    b[e] = (__bf16)(2e-3f * (float)e);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[blockIdx.x * kProbeThreads + threadIdx.x] = s;   // keeps the products live
}

constexpr int kReadBlocks = 2048;     // 8 blocks of 256 threads per CU: full occupancy
constexpr int kReadThreads = 256;

__global__ __launch_bounds__(kReadThreads) void hbm_read_kernel(const u32x4* src, int64_t n16,
                                                                uint32_t* sink) {
  const int64_t stride = (int64_t)gridDim.x * kReadThreads;
  int64_t i = (int64_t)blockIdx.x * kReadThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  sink[blockIdx.x * kReadThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

// Floats the sink buffer must hold.
int64_t vmla_probe_sink_floats(void) { return (int64_t)kProbeBlocks * kProbeThreads; }

// Dense bf16 flops of one probe launch of iters loop trips.
double vmla_probe_mfma_flops(int32_t iters) {
  return (double)kProbeBlocks * (kProbeThreads / 64) * (double)iters * kChains * (2.0 * 32 * 32 * 16);
}

// Launch the probe on stream (NULL: the default stream). sink: device floats,
// at least vmla_probe_sink_floats(); iters >= 1. Returns 0, -1 for bad
// arguments, -7 for a failed launch.
int32_t vmla_probe_mfma_bf16(float* sink, int32_t iters, void* stream) {
  if (!sink || iters < 1) return -1;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// 32-bit words the sink of vmla_probe_hbm_read must hold.
int64_t vmla_probe_read_sink_words(void) { return (int64_t)kReadBlocks * kReadThreads; }

// Read bytes (a positive multiple of 16) from the 16-byte aligned device
// buffer src on stream. Returns 0, -1 for bad arguments, -7 for a failed launch.
int32_t vmla_probe_hbm_read(const void* src, int64_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink || bytes <= 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return -1;
  hipLaunchKernelGGL(hbm_read_kernel, dim3(kReadBlocks), dim3(kReadThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

}  // extern "C"
