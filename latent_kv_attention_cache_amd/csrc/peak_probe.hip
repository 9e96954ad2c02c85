// Matrix-core peak probe: the measured second reference line of the bf16
// roofline. Every SIMD runs waves that issue independent back-to-back
// v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic inside
// the loop, so the launch time is the sustained dense bf16 MFMA rate of the
// chip at the clock it holds under that load. Not part of the library's C ABI:
// built into its own libvmla_probe.so and used by bench.py only.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

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

}  // extern "C"
