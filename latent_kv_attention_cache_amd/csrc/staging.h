// Global -> LDS staging helpers for the projection kernels (query prologue and
// cache append): multi-stage pipelines over the d_model contraction.
//
// A stage holds a 64-deep slice of the K dimension:
//   A tile: rows [m0, m0 + MT) x [k0, k0 + 64) of a row-major matrix (x); each
//           row is 64 bf16 = 8 chunks of 16 B and chunk c of row r is stored at
//           chunk position c ^ swz_a(r), so the row-wise 16-byte operand reads
//           of 16 consecutive rows hit distinct banks.
//   B tile: rows [k0, k0 + 64) x [n0, n0 + NT) of a row-major weight [K][ld];
//           each row is NT bf16 and its 64-byte column blocks are XOR-permuted
//           by swz_b<NT>(k), so the transpose reads of 4 consecutive rows hit
//           distinct banks (NT = 128: 256-byte rows; NT = 192: 384-byte rows;
//           NT = 32: 64-byte rows, no permutation needed).
// bf16 sources are copied with 16-byte LDS-DMA loads (no VGPR staging); fp32
// sources are converted to bf16 through registers into the same layout.
#pragma once
#include <type_traits>

#include "device_common.h"

namespace vmla {

constexpr int kStageK = 64;

__device__ __forceinline__ int swz_a(int r) { return (r ^ (r >> 3)) & 7; }

template <int NT>
__device__ __forceinline__ int swz_b(int k) {
  if constexpr (NT == 128) return k & 3;
  else if constexpr (NT == 192) return (k >> 1) & 1;
  else return 0;
}

// 16-byte LDS-DMA load: lane i's 16 bytes from base + voff (bytes; base
// wave-uniform) land at LDS byte address lds_addr + 16 i (lds_addr
// wave-uniform). Inline assembly so the compiler does not serialize unrelated
// LDS reads behind it; callers wait with s_waitcnt vmcnt. No register output.
__device__ __forceinline__ void dma16_lds(const void* base, uint32_t voff, uint32_t lds_addr) {
  // the base is wave-uniform; take it through readfirstlane so it is an SGPR pair
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint64_t sp = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(p >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)p);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(reinterpret_cast<const void*>(sp)),
                  "s"(__builtin_amdgcn_readfirstlane(lds_addr)) : "memory");
}

__device__ __forceinline__ uint32_t lds_u32(const bf16_t* p) {
  return (uint32_t)(uintptr_t)(VMLA_LDS const bf16_t*)p;
}

// One wave-wide 1 KB load (index n) of an A tile with MT rows. Rows past n_rows
// are clamped to the last row (finite data; those results are discarded).
template <typename T>
__device__ __forceinline__ void stage_a_load(bf16_t* dst, const T* src, int ld, int m0, int n_rows,
                                             int k0, int n, int lane) {
  const int slot = 64 * n + lane;                    // 16-byte slot in the tile
  const int r = slot >> 3;
  const int c = (slot & 7) ^ swz_a(r);
  const int row = min(m0 + r, n_rows - 1);
  if constexpr (std::is_same_v<T, bf16_t>) {
    dma16_lds(src, (uint32_t)(((size_t)row * ld + k0 + 8 * c) * sizeof(T)), lds_u32(dst + 512 * n));
  } else {
    *reinterpret_cast<uint4*>(dst + 8 * slot) = load8_bf16<T>(src + (size_t)row * ld + k0 + 8 * c);
  }
}

// One wave-wide 1 KB load (index n) of a B tile of width NT.
template <typename T, int NT>
__device__ __forceinline__ void stage_b_load(bf16_t* dst, const T* src, int ld, int n0, int k0, int n,
                                             int lane) {
  constexpr int kChunksRow = NT / 8;
  const int slot = 64 * n + lane;
  const int k = slot / kChunksRow;
  const int cpos = slot - k * kChunksRow;            // stored chunk position
  const int col = ((((cpos >> 2) ^ swz_b<NT>(k)) << 2) | (cpos & 3)) * 8;
  if constexpr (std::is_same_v<T, bf16_t>) {
    dma16_lds(src, (uint32_t)(((size_t)(k0 + k) * ld + n0 + col) * sizeof(T)), lds_u32(dst + 512 * n));
  } else {
    *reinterpret_cast<uint4*>(dst + 8 * slot) = load8_bf16<T>(src + (size_t)(k0 + k) * ld + n0 + col);
  }
}

// Byte offsets of one lane's 16 bytes in load n, relative to the stage's first
// element (A tile: &src[0][k0] with rows from m0; B tile: &src[k0][n0]). They do
// not depend on the stage, so a pipeline computes them once and only moves a
// scalar base pointer from stage to stage (bf16 sources).
__device__ __forceinline__ uint32_t stage_a_voff(int ld, int m0, int n_rows, int n, int lane) {
  const int slot = 64 * n + lane;
  const int r = slot >> 3;
  const int c = (slot & 7) ^ swz_a(r);
  const int row = min(m0 + r, n_rows - 1);
  return (uint32_t)(row * ld + 8 * c) * 2u;
}

template <int NT>
__device__ __forceinline__ uint32_t stage_b_voff(int ld, int n, int lane) {
  constexpr int kChunksRow = NT / 8;
  const int slot = 64 * n + lane;
  const int k = slot / kChunksRow;
  const int cpos = slot - k * kChunksRow;
  const int col = ((((cpos >> 2) ^ swz_b<NT>(k)) << 2) | (cpos & 3)) * 8;
  return (uint32_t)(k * ld + col) * 2u;
}

// Row-wise A operand (8 bf16) of MFMA 32x32x16: row r, K step ks of the stage.
__device__ __forceinline__ bf16x8 a_frag(const bf16_t* tile, int r, int ks, int half) {
  return lds_row8(tile + 64 * r + 8 * ((2 * ks + half) ^ swz_a(r)));
}

// Transposed B operand (8 bf16) of MFMA 32x32x16: lane l receives
// B[16 ks + 8 half + e][n0 + l%32], e = 0..7 (n0 a multiple of 32).
template <int NT>
__device__ __forceinline__ bf16x8 b_frag(const bf16_t* tile, int ks, int n0, int lane) {
  const int half = lane >> 5;
  const int j = lane & 15;
  const int nin = (lane & 16) + 4 * (j & 3);         // column within the 32-wide block
  const int k = 16 * ks + 8 * half + (j >> 2);
  const int blk = n0 >> 5;
  const bf16x4 lo = lds_tr4(tile + k * NT + ((blk ^ swz_b<NT>(k)) << 5) + nin);
  const bf16x4 hi = lds_tr4(tile + (k + 4) * NT + ((blk ^ swz_b<NT>(k + 4)) << 5) + nin);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// s_waitcnt vmcnt(stages * kLoads) for stages in {0, 1, 2}.
template <int kLoads>
__device__ __forceinline__ void wait_stages(int stages) {
  if (stages <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (stages == 1) asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kLoads) : "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * kLoads) : "memory");
}

}  // namespace vmla
