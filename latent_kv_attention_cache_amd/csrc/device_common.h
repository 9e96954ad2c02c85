// Device helpers shared by the gfx950 kernels of the latent-KV attention library.
//
// Matrix-core conventions (CDNA4 bf16 MFMA, checked by an in-bounds lane probe):
//  * v_mfma_f32_32x32x16_bf16: lane l supplies A[l%32][8*(l/32) + e] and
//    B[8*(l/32) + e][l%32], e = 0..7; result register r of lane l holds
//    D[8*(r/4) + 4*(l/32) + r%4][l%32].
//  * ds_read_b64_tr_b16: inside each group of 16 lanes, lane i receives element
//    i%4 of the 8-byte row that lane 4*r + i/4 addressed, r = 0..3. With lane j
//    of the group pointing at M[k0 + j/4][n0 + 4*(j%4)] of a row-major tile,
//    lane i receives M[k0 + r][n0 + i], r = 0..3: a transposed operand read.
//  * v_permlane32_swap(x, x) returns (r0, r1) such that {r0, r1} = {x[l], x[l^32]}
//    in every lane l.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vmla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t bf16_t;   // bf16 storage in global memory

#define VMLA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Transposed 4-element read (see the header comment).
__device__ __forceinline__ bf16x4 lds_tr4(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((bf16x4 VMLA_LDS*)(p));
}

// Operand fragment of a 32-wide MFMA operand read transposed out of a row-major
// LDS tile M[k][n] (leading dimension ld elements): lane l receives
// M[ka + e][n0 + l%32] for e = 0..3 and M[kb + e - 4][n0 + l%32] for e = 4..7,
// where ka / kb are the per-half row bases the caller computes for lane half l/32.
__device__ __forceinline__ bf16x8 lds_tr8(const bf16_t* tile, int ld, int ka, int kb, int n0,
                                           int lane) {
  const int j = lane & 15;
  const int nsub = (lane & 16);               // 16 * ((lane / 16) % 2)
  const int col = n0 + nsub + 4 * (j & 3);
  bf16x4 lo = lds_tr4(tile + (ka + (j >> 2)) * ld + col);
  bf16x4 hi = lds_tr4(tile + (kb + (j >> 2)) * ld + col);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 lds_row8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return (uint32_t)f2bf(a) | ((uint32_t)f2bf(b) << 16);
}

// Load 8 consecutive elements of T as 8 bf16 (16 bytes); T is bf16_t or float.
template <typename T> __device__ __forceinline__ uint4 load8_bf16(const T* p);
template <> __device__ __forceinline__ uint4 load8_bf16<bf16_t>(const bf16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
template <> __device__ __forceinline__ uint4 load8_bf16<float>(const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  return make_uint4(pack2(a.x, a.y), pack2(a.z, a.w), pack2(b.x, b.y), pack2(b.z, b.w));
}

template <typename T> __device__ __forceinline__ T from_f32(float f);
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return f2bf(f); }
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }

__device__ __forceinline__ float bf2f(bf16_t v) {
  return __uint_as_float((uint32_t)v << 16);
}

// Exchange with lane l^1 (the other channel of a RoPE pair).
__device__ __forceinline__ float swap_adjacent(float v) {
  // DPP quad_perm [1,0,3,2]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}

// q = n / d and *rem = n % d for 0 <= n < 2^24 and 1 <= d < 2^24, with
// inv_d = 1 / d rounded to float: the float estimate is within 2 of the
// quotient, and two correction steps each way make the result exact. Replaces
// the long integer-division sequence in per-row position arithmetic.
__device__ __forceinline__ int div_small(int n, int d, float inv_d, int* rem) {
  int q = (int)((float)n * inv_d);
  int r = n - q * d;
  if (r < 0) { --q; r += d; }
  if (r < 0) { --q; r += d; }
  if (r >= d) { ++q; r -= d; }
  if (r >= d) { ++q; r -= d; }
  *rem = r;
  return q;
}

// sin and cos of the angle pos * rate for a rate given in revolutions per
// position step as a 64-bit binary fraction (hi:lo) = rate * 2^64. The
// fractional revolution of the product is taken in integer arithmetic, exact
// mod 1 up to the rate's own rounding (< pos * 2^-64 revolutions), then
// truncated to 32 bits, so the angle error is below 2^-32 revolutions at any
// position; v_sin_f32 / v_cos_f32 take their input in revolutions.
__device__ __forceinline__ void sincos_rev(int pos, uint32_t lo, uint32_t hi, float* s, float* c) {
  const uint32_t p = (uint32_t)pos;
  const uint32_t frac = __umulhi(p, lo) + p * hi;        // bits 32..63 of pos * rate, mod 2^64
  const float r = (float)frac * 2.3283064365386963e-10f;  // * 2^-32: [0, 1]
  *s = __builtin_amdgcn_sinf(r);
  *c = __builtin_amdgcn_cosf(r);
}

// RoPE rates of pair j0 + 2 g for the lane's 16-lane group g (0..3), with
// j0 uniform across the wave, from a by-value kernel-argument table (arrays
// rev_lo, rev_hi, axis). The four candidates are read with scalar loads and
// each lane keeps its own: indexing a kernel argument with a per-lane index
// compiles to per-lane loads from the kernel-argument segment, whose latency
// then sits in the epilogue's critical path.
template <typename Table>
__device__ __forceinline__ void rope_rate_by_group(const Table& t, int j0, int g, uint32_t* lo,
                                                   uint32_t* hi, int* ax) {
  // readfirstlane on each loaded candidate keeps the compiler from turning
  // "select after load" back into a per-lane load of the selected entry
  const int j = __builtin_amdgcn_readfirstlane(j0);
  uint32_t l = __builtin_amdgcn_readfirstlane(t.rev_lo[j]), h = __builtin_amdgcn_readfirstlane(t.rev_hi[j]);
  int x = __builtin_amdgcn_readfirstlane(t.axis[j]);
#pragma unroll
  for (int k = 1; k < 4; ++k) {
    const uint32_t lk = __builtin_amdgcn_readfirstlane(t.rev_lo[j + 2 * k]);
    const uint32_t hk = __builtin_amdgcn_readfirstlane(t.rev_hi[j + 2 * k]);
    const int xk = __builtin_amdgcn_readfirstlane(t.axis[j + 2 * k]);
    if (g == k) {
      l = lk;
      h = hk;
      x = xk;
    }
  }
  *lo = l;
  *hi = h;
  *ax = x;
}

__device__ __forceinline__ float max_across_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_across_halves(float v) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace vmla
