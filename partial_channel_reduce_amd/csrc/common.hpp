// Shared device-side definitions for the gfx950 (CDNA4) kernels of the
// partial channel-reduce library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace caat {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 bits -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Non-temporal 16-byte global store: streamed outputs are not re-read by the
// kernel that writes them, so keep them from evicting reusable operand lines.
__device__ __forceinline__ void st16_nt(void* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

// LDS tiles hold operands as [row][64 k] bf16 rows of 128 bytes, i.e. eight
// 16-byte k-chunks per row.  The chunk index is XOR-swizzled with a function of
// the row so that (a) the MFMA operand reads (32 consecutive rows, one chunk)
// and (b) the transposing writes (rows 8 apart, one chunk) both spread over
// all 32 banks.
__device__ __forceinline__ int lds_swz(int row) { return (row ^ (row >> 3)) & 7; }
__device__ __forceinline__ int lds_off(int row, int chunk) {  // in bf16 elements
  return row * 64 + ((chunk ^ lds_swz(row)) << 3);
}

// 8x8 bf16 transpose held in registers: r[i] holds 8 consecutive columns of
// row i; on return o[j] holds column j as 8 consecutive rows.
__device__ __forceinline__ void transpose8x8(const u32x4 r[8], u32x4 o[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const uint32_t a = r[2 * d][j >> 1];
      const uint32_t b = r[2 * d + 1][j >> 1];
      o[j][d] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
    }
  }
}

// Block-id remap for 8-XCD parts: consecutive hardware block ids land on
// different XCDs (round robin), so hand each XCD a contiguous range of logical
// tiles; tiles that share operand rows then share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  constexpr int kXcd = 8;
  if (nblocks % kXcd != 0) return bid;
  return (bid % kXcd) * (nblocks / kXcd) + bid / kXcd;
}

}  // namespace caat
