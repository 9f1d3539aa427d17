// The step after the partial channel-reduce in the Llama-family blocks the
// CAAT-Net paper trains: each rank adds its own (now rank-specific)
// activation to its own residual stream and RMS-normalises the result.
//   Rn[t,m,:] = bf16(R[t,m,:] + Z[t,m,:])
//   N[t,m,:]  = bf16(Rn * gamma / sqrt(mean_c Rn^2 + eps))   (fp32 arithmetic)
#pragma once

#include "common.hpp"
#include "reduce_kernels.hpp"

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
// before it is written, by the same thread.  Every load of the thread is
// issued before its first store (the compiler may not move a load of R past
// a store to Rout, which may alias it), and all four streams bypass the
// caches' reuse (non-temporal): nothing here is read twice.
template <int KV>
__global__ void __launch_bounds__(kNormThreads)
pcr_residual_rmsnorm_kernel(const uint16_t* __restrict__ Z, const uint16_t* R, const uint16_t* __restrict__ gamma,
                            uint16_t* Rout, uint16_t* __restrict__ N, int H, float eps) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hv = H / 8;
  const long long base = (long long)blockIdx.x * H;
  u32x4 zv[KV], rn[KV];
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    const int v = tid + kNormThreads * i;
    if (v < hv) {
      zv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Z + base + v * 8));
      rn[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(R + base + v * 8));
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    const int v = tid + kNormThreads * i;
    if (v < hv) {
      const u32x4 z = zv[i], r = rn[i];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float lo = bf16_lo(z[d]) + bf16_lo(r[d]);
        const float hi = bf16_hi(z[d]) + bf16_hi(r[d]);
        rn[i][d] = pack_bf16x2(lo, hi);
        const float a = bf16_lo(rn[i][d]), b = bf16_hi(rn[i][d]);
        ss += a * a;
        ss += b * b;
      }
      st16_nt(Rout + base + v * 8, rn[i]);
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
      st16_nt(N + base + v * 8, o);
    }
  }
}

// ---- the partial channel-reduce with the residual update and norm in its
// epilogue ---------------------------------------------------------------------
// For per-rank bf16 activations Y[T,M,H] (the partial products before the
// reduce), one workgroup per token row m reads that row of every rank,
// forms Z_t (synced channels: the fp32 sum over the ranks in ascending order,
// rounded once to bf16; local channels: Y_t), and writes only
//   Rout[t,m,:] = bf16(R[t,m,:] + Z_t)   and   N[t,m,:] = RMS-normalised Rout row
// for every rank t; Z itself never goes to memory.  The arithmetic and its
// order are those of the reduce kernel followed by pcr_residual_rmsnorm_kernel
// (same thread layout: vectors tid + 256 i), so the results are the same bits
// as that two-kernel chain.
// TC > 0: T == TC <= 8 and the Y row is kept in registers between the sum
// and the epilogue; TC == 0: any T, ranks taken four at a time and the Y row
// read again from the cache.
template <int KV, int TC>
__global__ void __launch_bounds__(kNormThreads)
pcr_reduce_residual_rmsnorm_kernel(const uint16_t* __restrict__ Y, const uint8_t* __restrict__ mask,
                                   const uint16_t* R, const uint16_t* __restrict__ gamma, uint16_t* Rout,
                                   uint16_t* __restrict__ N, int T_rt, int H, long long mh, float eps,
                                   uint32_t groups) {
  constexpr int G = TC > 0 ? TC : 4;  // ranks normalised together
  const int T = TC > 0 ? TC : T_rt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hv = H / 8;
  // token row m in every rank slice (rows taken from `groups` regions in
  // turn, as in the reduce kernels)
  const long long row = (long long)reduce_block(groups) * H;
  __shared__ float wsum[kNormThreads / 64][G];
  u32x4 sel[KV], sv[KV];
  u32x4 yk[TC > 0 ? TC : 1][KV];
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    const int v = tid + kNormThreads * i;
    if (v < hv) {
      const u32x2 mk = *reinterpret_cast<const u32x2*>(mask + v * 8);
      sel[i] = expand_mask8(mk[0], mk[1]);
    }
  }
  // The synced sums: fp32, ascending rank order, starting from rank 0's value.
  float sacc[KV][8];
  if constexpr (TC > 0) {
#pragma unroll
    for (int t = 0; t < TC; ++t)
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const int v = tid + kNormThreads * i;
        if (v < hv) yk[t][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Y + t * mh + row + v * 8));
      }
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      bf16x8_to_f32(yk[0][i], sacc[i]);
#pragma unroll
      for (int t = 1; t < TC; ++t) {
        float f[8];
        bf16x8_to_f32(yk[t][i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) sacc[i][e] += f[e];
      }
    }
  } else {
    // Ranks eight at a time, every load of a group in flight together; the
    // sum keeps ascending rank order.
    for (int t0 = 0; t0 < T; t0 += 8)
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const int v = tid + kNormThreads * i;
        if (v < hv) {
          u32x4 g[8];
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (t0 + k < T) g[k] = ld16(Y + (t0 + k) * mh + row + v * 8);
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (t0 + k < T) {
              float f[8];
              bf16x8_to_f32(g[k], f);
#pragma unroll
              for (int e = 0; e < 8; ++e) sacc[i][e] = t0 + k == 0 ? f[e] : sacc[i][e] + f[e];
            }
        }
      }
  }
#pragma unroll
  for (int i = 0; i < KV; ++i)
#pragma unroll
    for (int d = 0; d < 4; ++d) sv[i][d] = pack_bf16x2(sacc[i][2 * d], sacc[i][2 * d + 1]);

  for (int g0 = 0; g0 < T; g0 += G) {
    u32x4 rn[G][KV];
    float ss[G];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      ss[j] = 0.f;
      const int t = g0 + j;
      if (t < T) {
#pragma unroll
        for (int i = 0; i < KV; ++i) {
          const int v = tid + kNormThreads * i;
          if (v < hv) {
            const long long off = t * mh + row + v * 8;
            u32x4 y;
            if constexpr (TC > 0)
              y = yk[j][i];
            else
              y = ld16(Y + off);
            const u32x4 z = (sv[i] & sel[i]) | (y & ~sel[i]);
            const u32x4 r = ld16(R + off);
#pragma unroll
            for (int d = 0; d < 4; ++d) {
              const float lo = bf16_lo(z[d]) + bf16_lo(r[d]);
              const float hi = bf16_hi(z[d]) + bf16_hi(r[d]);
              rn[j][i][d] = pack_bf16x2(lo, hi);
              const float a = bf16_lo(rn[j][i][d]), b = bf16_hi(rn[j][i][d]);
              ss[j] += a * a;
              ss[j] += b * b;
            }
            st16_nt(Rout + off, rn[j][i]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) ss[j] += __shfl_xor(ss[j], o, 64);
      if (lane == 0) wsum[wave][j] = ss[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int t = g0 + j;
      if (t < T) {
        float total = wsum[0][j];
#pragma unroll
        for (int w = 1; w < kNormThreads / 64; ++w) total += wsum[w][j];
        const float scale = 1.0f / sqrtf(total / (float)H + eps);
#pragma unroll
        for (int i = 0; i < KV; ++i) {
          const int v = tid + kNormThreads * i;
          if (v < hv) {
            const u32x4 g = ld16(gamma + v * 8);
            u32x4 o;
#pragma unroll
            for (int d = 0; d < 4; ++d)
              o[d] = pack_bf16x2(bf16_lo(rn[j][i][d]) * scale * bf16_lo(g[d]),
                                 bf16_hi(rn[j][i][d]) * scale * bf16_hi(g[d]));
            st16_nt(N + t * mh + row + v * 8, o);
          }
        }
      }
    }
    __syncthreads();  // wsum is rewritten by the next group
  }
}

}  // namespace caat
