// Decode-shaped forward (M <= 32 tokens): the same result as the fused forward,
// organised for weight streaming.  The layer then reads ~Kr*H*T*2 bytes of
// weights once and does almost no arithmetic per byte, so the grid is spread
// over (n-block, rank) pairs to keep enough weight loads in flight, and the
// cross-rank sum of the synced channels is finished by whichever workgroup of
// an n-block arrives last (it sums the T per-rank partials in ascending rank
// order, so the result does not depend on arrival order).
#pragma once

#include "gemm_core.hpp"

namespace caat {

constexpr int kDecMaxM = 32;  // rows of one 32x32 MFMA block
constexpr int kDecBN = 64;    // channels per workgroup
constexpr int kDecKC = 256;   // contraction rows staged per iteration

// Workspace layout for the decode path: [counters: one u32 per n-block,
// padded to 256 B][partials: fp32 [T][M][H]].
__host__ __device__ inline size_t dec_counter_bytes(int H) {
  const size_t n = (size_t)((H + kDecBN - 1) / kDecBN) * 4;
  return (n + 255) & ~(size_t)255;
}

__device__ __forceinline__ int dec_lds_off(int row, int chunk) {  // [64 rows][256 k] bf16
  return row * kDecKC + ((chunk ^ lds_swz(row)) << 3);
}

__global__ void __launch_bounds__(kGemmThreads)
rowpar_pcr_decode_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                         const uint8_t* __restrict__ mask, uint16_t* __restrict__ out,
                         uint32_t* __restrict__ counters, float* __restrict__ partial,
                         int T, int M, int Kr, int H) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[kDecBN * kDecKC];  // 32 KiB
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nblocks = (H + kDecBN - 1) / kDecBN;
  const int nb = blockIdx.x % nblocks;
  const int t = blockIdx.x / nblocks;
  const int n0 = nb * kDecBN;
  const long long MK = (long long)M * Kr, KH = (long long)Kr * H, MH = (long long)M * H;
  const uint16_t* Xt = X + t * MK;
  const uint16_t* Wt = W + t * KH;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  // Each thread owns one 8(k) x 8(n) block of the 256 x 64 weight chunk.
  const int bn = tid % (kDecBN / 8), bk = tid / (kDecBN / 8);
  const int wcol = min(n0 + bn * 8, H - 8);
  u32x4 wv[8];
  auto load_w = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int k = k0 + bk * 8 + i;
      wv[i] = (k < Kr) ? ld16(Wt + (long long)k * H + wcol) : zero;
    }
  };
  auto store_w = [&]() {
    u32x4 o[8];
    transpose8x8(wv, o);
#pragma unroll
    for (int j = 0; j < 8; ++j) st16(smem + dec_lds_off(bn * 8 + j, bk), o[j]);
  };

  f32x16 acc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[j][e] = 0.f;

  const int arow = lane & 31;
  const bool arow_ok = arow < M;
  const int nchunks = (Kr + kDecKC - 1) / kDecKC;
  load_w(0);
  for (int c = 0; c < nchunks; ++c) {
    const int k0 = c * kDecKC;
    __syncthreads();  // previous chunk's LDS reads are done
    store_w();
    if (c + 1 < nchunks) load_w(k0 + kDecKC);
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kk = wave * 64 + ks * 16 + (lane >> 5) * 8;  // within the chunk
      const int k = k0 + kk;
      const u32x4 a = (arow_ok && k < Kr) ? ld16(Xt + (long long)arow * Kr + k) : zero;
      const int ch = (wave * 64 + ks * 16) / 8 + (lane >> 5);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 b = ld16(smem + dec_lds_off(j * 32 + (lane & 31), ch));
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), acc[j], 0, 0, 0);
      }
    }
  }

  // Sum the four waves' partial products (fixed order, through LDS).
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);  // [4 waves][32 rows][64 cols] = 32 KiB
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e)
      red[(wave * 32 + acc_row(e, lane)) * kDecBN + j * 32 + (lane & 31)] = acc[j][e];
  __syncthreads();

  const int cl = tid % kDecBN;  // channel within the block
  const int c = n0 + cl;
  const bool c_ok = c < H;
  const bool synced = c_ok && mask[c] != 0;
  for (int m = tid / kDecBN; m < M; m += kGemmThreads / kDecBN) {
    float y = red[(0 * 32 + m) * kDecBN + cl];
    y += red[(1 * 32 + m) * kDecBN + cl];
    y += red[(2 * 32 + m) * kDecBN + cl];
    y += red[(3 * 32 + m) * kDecBN + cl];
    if (!c_ok) continue;
    if (synced)
      partial[t * MH + (long long)m * H + c] = y;
    else
      out[t * MH + (long long)m * H + c] = f32_to_bf16(y);
  }

  // Last of the T workgroups of this n-block finishes the synced channels.
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const uint32_t prev = atomicAdd(counters + nb, 1u);
    s_last = (prev == (uint32_t)(T - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (synced) {
    for (int m = tid / kDecBN; m < M; m += kGemmThreads / kDecBN) {
      const long long off = (long long)m * H + c;
      float s = __builtin_nontemporal_load(partial + off);
      for (int u = 1; u < T; ++u) s += __builtin_nontemporal_load(partial + u * MH + off);
      const uint16_t v = f32_to_bf16(s);
      for (int u = 0; u < T; ++u) out[u * MH + off] = v;
    }
  }
  if (tid == 0) atomicExch(counters + nb, 0u);  // leave the counter zeroed for the next call
}

}  // namespace caat
