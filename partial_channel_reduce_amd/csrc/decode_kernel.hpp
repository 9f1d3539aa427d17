// Decode-shaped forward (M <= 32 tokens): the same result as the fused
// forward, organised for weight streaming.  With so few tokens the layer reads
// ~T*Kr*H*2 bytes of weights once and does almost no arithmetic per byte, so
// it runs as two kernels laid out for HBM streaming:
//
//   rowpar_pcr_decode_kernel: one workgroup per (rank t, 64-channel block), so
//     every weight row piece it reads is one whole 128-byte line.  Its 4 waves
//     split the contraction; each streams 32-row x 64-channel stages straight
//     into LDS (buffer loads, 3 stages in flight per wave) and feeds them to
//     16x16x32 bf16 MFMAs through gfx950's LDS transpose read, with the token
//     rows of X_t read into A fragments alongside.  The waves' partial sums
//     are added in wave order through LDS; local channels are written to
//     out[t] as bf16, synced channels leave their fp32 value in the workspace.
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
constexpr int kDecDepth = 4;     // stage slots per wave: one being read, three in flight

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

template <int NB>  // MFMA row blocks of 16 tokens: 1 (M <= 16) or 2
__global__ void __launch_bounds__(kDecThreads)
rowpar_pcr_decode_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                         const uint8_t* __restrict__ mask, uint16_t* __restrict__ out,
                         float* __restrict__ partial, int T, int M, int Kr, int H) {
  constexpr int SE = kDecStage * kDecCols;  // elements per stage (4 KiB)
  __shared__ __attribute__((aligned(16))) uint16_t lds[kDecWaves * kDecDepth * SE];  // 64 KiB
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

  // Weight DMA: an instruction moves 8 k-rows x 64 channels (1 KiB); this
  // lane's slot is k-row lane/8, stored chunk lane%8.  Rows past Kr read as
  // zero (they only occur past the last wave's end).
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(W + t * KH, (uint32_t)(KH * 2));
  const int wrow = lane >> 3;
  const int wvoff = (wrow * H + (((lane & 7) ^ ((wrow & 3) << 1)) << 3)) * 2;
  uint16_t* slots = lds + wave * kDecDepth * SE;
  auto issue_w = [&](int st) {
    uint16_t* tile = slots + (st % kDecDepth) * SE;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int soff = __builtin_amdgcn_readfirstlane(((kbeg + st * kDecStage + 8 * i) * H + n0) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wrs, (lds_void_t*)(tile + 8 * i * kDecCols), 16, wvoff, soff, 0, 0);
    }
  };
  // A fragments: token row xr (+16 for block 1), k offset xk within the stage.
  // Rows past M and k past this wave's range are pointed beyond the end of the
  // X_t buffer, so the load itself returns zeros: every lane always issues the
  // same loads (the vmcnt accounting below relies on it) and nothing waits on
  // a select.
  const int xr = lane & 15, xk = (lane >> 4) * 8;
  const uint32_t xbytes = (uint32_t)(MK * 2);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(Xt, xbytes);
  auto load_x = [&](int st, u32x4 (&x)[NB]) {
    const int k = kbeg + st * kDecStage + xk;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int m = xr + 16 * b;
      const uint32_t voff = (m < M && k < kend) ? (uint32_t)(m * Kr + k) * 2u : xbytes;
      x[b] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, voff, 0, 0));
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
  auto step = [&](int st, const u32x4 (&xuse)[NB], u32x4 (&xnext)[NB]) {
    issue_w(st + kDecDepth - 1);  // stages past the end read zeros
    load_x(st + kDecDepth - 1, xnext);
    wait_vmcnt<(kDecDepth - 1) * (4 + NB)>();  // stage st has landed
    const uint16_t* tile = slots + (st % kDecDepth) * SE;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4 b;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * g + 4 * h + s4;
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + dec_off(row, j * 16 + 4 * u4)));
        const u32x2 w2 = __builtin_bit_cast(u32x2, v);
        b[2 * h] = w2[0];
        b[2 * h + 1] = w2[1];
      }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
        acc[bb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(xuse[bb]), as_bf16x8(b), acc[bb][j], 0, 0, 0);
    }
    // This slot is refilled by the next step's issue: finish reading it.
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };

  // Token fragments for stages st..st+3 rotate through four register sets by
  // unrolling the stage loop four times (copies would wait on the loads).
  u32x4 x0[NB], x1[NB], x2[NB], x3[NB];
  issue_w(0);
  load_x(0, x0);
  issue_w(1);
  load_x(1, x1);
  issue_w(2);
  load_x(2, x2);
  for (int st = 0; st < nst; st += 4) {
    step(st, x0, x3);
    if (st + 1 >= nst) break;
    step(st + 1, x1, x0);
    if (st + 2 >= nst) break;
    step(st + 2, x2, x1);
    if (st + 3 >= nst) break;
    step(st + 3, x3, x2);
  }
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
