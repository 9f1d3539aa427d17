// Decode-shaped forward (M <= 32 tokens): the same result as the fused
// forward, organised for weight streaming.  With so few tokens the layer reads
// ~T*Kr*H*2 bytes of weights once and does almost no arithmetic per byte, so
// it runs as two kernels laid out for HBM streaming:
//
//   rowpar_pcr_decode_kernel: one workgroup per (rank t, 64-channel block), so
//     every weight row piece it reads is one whole 128-byte line.  Its 4 waves
//     split the contraction; each streams 32-row x 64-channel weight stages
//     and the matching 32 columns of X_t's token rows straight into LDS
//     (buffer loads, 3 stages in flight per wave) and feeds them to 16x16x32
//     bf16 MFMAs, the weights through gfx950's LDS transpose read.  The
//     waves' partial sums are added in wave order through LDS; local channels
//     are written to out[t] as bf16, synced channels leave their fp32 value in
//     the workspace.
//
//   decode_sync_sum_kernel: for each synced (token, channel) the T fp32 values
//     are added in ascending rank order and the one bf16 result is written to
//     every rank.  The kernel boundary orders it after the first kernel; no
//     atomics or device-wide fences are involved.
#pragma once

#include "gemm_core.hpp"

namespace caat {

constexpr int kDecMaxM = 32;     // two 16-row MFMA blocks
constexpr int kDecCols = 64;     // channels per workgroup: one 128-byte line per row
constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecStage = 32;    // contraction rows per stage (one MFMA k-step)

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// LDS stage layout [32 k][64 channels], 128-byte rows; 16-byte chunks XOR
// swizzled by 2*(k%4) so the 4 k-rows of a transpose read hit distinct banks.
__device__ __forceinline__ int dec_off(int k, int ch) { return k * kDecCols + (((ch >> 3) ^ ((k & 3) << 1)) << 3) + (ch & 7); }

// X stage layout [16*NB token rows][32 k], 64-byte rows; 16-byte chunks XOR
// swizzled by (row / 4) % 4 so the 16 rows of an A-fragment read hit distinct
// banks.
__device__ __forceinline__ int dec_xoff(int row, int ch) { return row * kDecStage + ((ch ^ ((row >> 2) & 3)) << 3); }

template <int NB>  // MFMA row blocks of 16 tokens: 1 (M <= 16) or 2
__global__ void __launch_bounds__(kDecThreads)
rowpar_pcr_decode_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                         const uint8_t* __restrict__ mask, uint16_t* __restrict__ out,
                         float* __restrict__ partial, int T, int M, int Kr, int H) {
  // Stage slots per wave: 4 (3 in flight) with one 16-token block, 3 with two,
  // so that a workgroup needs at most 80 KiB of LDS and two fit on a CU.
  constexpr int kDecDepth = NB == 1 ? 4 : 3;
  constexpr int SE = kDecStage * kDecCols;  // W elements per stage (4 KiB)
  constexpr int XE = 16 * NB * kDecStage;   // X elements per stage (1 or 2 KiB)
  constexpr int SLOT = SE + XE;
  constexpr int LDS = kDecWaves * kDecDepth * SLOT > kDecWaves * kDecMaxM * kDecCols * 2
                          ? kDecWaves * kDecDepth * SLOT
                          : kDecWaves * kDecMaxM * kDecCols * 2;  // stages, or the fp32 reduction area
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = (H + kDecCols - 1) / kDecCols;
  const int t = blockIdx.x / nb;
  const int n0 = (blockIdx.x - t * nb) * kDecCols;
  const long long MK = (long long)M * Kr, KH = (long long)Kr * H, MH = (long long)M * H;
  const uint16_t* Xt = X + t * MK;

  // This wave's share of the contraction: a multiple of 32 rows per wave.
  const int kq = (((Kr + kDecWaves - 1) / kDecWaves) + kDecStage - 1) / kDecStage * kDecStage;
  const int kbeg = min(Kr, wave * kq), kend = min(Kr, kbeg + kq);
  const int nst = (kend - kbeg + kDecStage - 1) / kDecStage;

  // Both operands are copied global -> LDS, 4 + NB wave instructions per
  // stage.  Weight rows past Kr and token rows past M, and X columns past this
  // wave's range, read as zero (out of the buffer's range).
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(W + t * KH, (uint32_t)(KH * 2));
  const int wrow = lane >> 3;
  const int wvoff = (wrow * H + (((lane & 7) ^ ((wrow & 3) << 1)) << 3)) * 2;
  const uint32_t xbytes = (uint32_t)(MK * 2);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(Xt, xbytes);
  const int xch = (lane & 3) ^ ((lane >> 4) & 3);  // logical k-chunk this lane copies
  uint16_t* slots = lds + wave * kDecDepth * SLOT;
  auto issue = [&](int st) {
    uint16_t* tile = slots + (st % kDecDepth) * SLOT;
    const int k0 = kbeg + st * kDecStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int soff = __builtin_amdgcn_readfirstlane(((k0 + 8 * i) * H + n0) * 2);
      dma16(wrs, tile + 8 * i * kDecCols, wvoff, soff);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int m = (lane >> 2) + 16 * b;
      const bool ok = m < M && k0 + xch * 8 < kend;
      const int voff = ok ? (m * Kr + xch * 8) * 2 : (int)xbytes;
      dma16(xrs, tile + SE + 16 * b * kDecStage, voff, __builtin_amdgcn_readfirstlane(k0 * 2));
    }
  };

  f32x4_t acc[NB][4];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[b][j][e] = 0.f;

  // tr-read addressing (16x16x32 B operand): lane 4s+u of 16-lane group g
  // names k-row 8g+4h+s and channels 4u..4u+3 of a 16-channel block.
  const int g = lane >> 4, s4 = (lane & 15) >> 2, u4 = lane & 3;
  auto step = [&](int st) {
    issue(st + kDecDepth - 1);  // stages past the end read zeros
    wait_vmcnt<(kDecDepth - 1) * (4 + NB)>();  // this wave's copies of stage st have landed
    const uint16_t* tile = slots + (st % kDecDepth) * SLOT;
    u32x4 xa[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) xa[b] = ld16(tile + SE + dec_xoff(16 * b + (lane & 15), lane >> 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 bv;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * g + 4 * h + s4;
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + dec_off(row, j * 16 + 4 * u4)));
        const u32x2 w2 = __builtin_bit_cast(u32x2, v);
        bv[2 * h] = w2[0];
        bv[2 * h + 1] = w2[1];
      }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
        acc[bb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xa[bb]), as_bf16x8(bv), acc[bb][j], 0, 0, 0);
    }
    // This slot is refilled by the next step's issue: finish reading it.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  for (int p = 0; p < kDecDepth - 1; ++p) issue(p);
  for (int st = 0; st < nst; ++st) step(st);
  wait_vmcnt<0>();
  __syncthreads();

  // Add the waves' partial products in wave order.  Accumulator layout
  // (16x16): channel 16j + lane%16, token rows 16b + 4*(lane/16) + e.
  float* red = reinterpret_cast<float*>(lds);  // [4 waves][32 tokens][64 channels] = 32 KiB
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        red[(wave * kDecMaxM + 16 * b + 4 * g + e) * kDecCols + 16 * j + (lane & 15)] = acc[b][j][e];
  __syncthreads();
  const int cl = tid % kDecCols, c = n0 + cl;
  if (c >= H) return;
  const bool synced = mask[c] != 0;
  for (int m = tid / kDecCols; m < M; m += kDecThreads / kDecCols) {
    float y = red[(0 * kDecMaxM + m) * kDecCols + cl];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) y += red[(w * kDecMaxM + m) * kDecCols + cl];
    const long long off = t * MH + (long long)m * H + c;
    if (synced)
      partial[off] = y;
    else
      out[off] = f32_to_bf16(y);
  }
}

// Synced channels: out[t][m][c] = bf16( sum_t partial[t][m][c] ), ascending t.
__global__ void __launch_bounds__(256)
decode_sync_sum_kernel(const float* __restrict__ partial, const uint8_t* __restrict__ mask,
                       uint16_t* __restrict__ out, int T, int M, int H) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M * H) return;
  const int c = i % H;
  if (mask[c] == 0) return;
  const long long MH = (long long)M * H;
  float s = partial[i];
  for (int t = 1; t < T; ++t) s += partial[t * MH + i];
  const uint16_t v = f32_to_bf16(s);
  for (int t = 0; t < T; ++t) out[t * MH + i] = v;
}

}  // namespace caat
