// The step after the partial channel-reduce in the Llama-family blocks the
// CAAT-Net paper trains: each rank adds its own (now rank-specific)
// activation to its own residual stream and RMS-normalises the result.
//   Rn[t,m,:] = bf16(R[t,m,:] + Z[t,m,:])
//   N[t,m,:]  = bf16(Rn * gamma / sqrt(mean_c Rn^2 + eps))   (fp32 arithmetic)
#pragma once

#include "common.hpp"

namespace caat {

constexpr int kNormThreads = 256;
constexpr int kNormMaxVecs = 4;  // 8-channel vectors per thread: H <= 8192

// One workgroup per token row (t, m).  Thread tid owns the 8-channel vectors
// tid + 256 i, i < KV, and keeps the rounded Rn values in registers between
// the two passes.  The row's sum of squares (over the rounded values, in
// fp32) is formed in a fixed order -- each thread over its vectors in order,
// a butterfly across the wave read from lane 0, then the four waves in
// order -- so every run gives the same bits.  R and Rout may be the same
// array (in-place update of the residual stream): each element is read
// before it is written, by the same thread.
template <int KV>
__global__ void __launch_bounds__(kNormThreads)
pcr_residual_rmsnorm_kernel(const uint16_t* __restrict__ Z, const uint16_t* R, const uint16_t* __restrict__ gamma,
                            uint16_t* Rout, uint16_t* __restrict__ N, int H, float eps) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hv = H / 8;
  const long long base = (long long)blockIdx.x * H;
  u32x4 rn[KV];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    const int v = tid + kNormThreads * i;
    if (v < hv) {
      const u32x4 z = ld16(Z + base + v * 8), r = ld16(R + base + v * 8);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float lo = bf16_lo(z[d]) + bf16_lo(r[d]);
        const float hi = bf16_hi(z[d]) + bf16_hi(r[d]);
        rn[i][d] = pack_bf16x2(lo, hi);
        const float a = bf16_lo(rn[i][d]), b = bf16_hi(rn[i][d]);
        ss += a * a;
        ss += b * b;
      }
      st16(Rout + base + v * 8, rn[i]);
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
  __shared__ float wsum[kNormThreads / 64];
  if (lane == 0) wsum[wave] = ss;
  __syncthreads();
  float total = wsum[0];
#pragma unroll
  for (int w = 1; w < kNormThreads / 64; ++w) total += wsum[w];
  const float scale = 1.0f / sqrtf(total / (float)H + eps);
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    const int v = tid + kNormThreads * i;
    if (v < hv) {
      const u32x4 g = ld16(gamma + v * 8);
      u32x4 o;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o[d] = pack_bf16x2(bf16_lo(rn[i][d]) * scale * bf16_lo(g[d]), bf16_hi(rn[i][d]) * scale * bf16_hi(g[d]));
      st16(N + base + v * 8, o);
    }
  }
}

}  // namespace caat
