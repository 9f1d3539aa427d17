// HBM-streaming kernels of the partial channel-reduce:
//   * the standalone reduce over per-rank activations Y[T,M,H] (fp32 or bf16),
//     which in bf16 also forms the backward's reduced gradient G from dZ.
//
// Definition (CAAT-Net paper, Introduction): only the hidden channels of the
// sync set S are summed over the T tensor-parallel ranks; the other channels
// keep each rank's own value.  Sums run in fp32 in ascending rank order,
// starting from rank 0's value, are formed once per (m, c) and written to every
// rank, so the synced channels are bit-identical across ranks.
#pragma once

#include "common.hpp"

namespace caat {

constexpr int kReduceThreads = 256;

// Workgroup -> row-block order.  When the ranks' slices lie a large power of
// two apart, the T addresses of one element fall on the same HBM channels,
// and workgroups that run together (consecutive indices) pile onto them.
// With `groups` = G > 1, consecutive workgroups take row blocks from G
// different regions of the rows (G = 2: the two halves; G = 8: eight
// regions), which spreads the concurrent accesses (measured on MI355X at
// 8 x 16384 x 4096: fp32 +13%, bf16 +18%).
__device__ __forceinline__ uint32_t reduce_block(uint32_t groups) {
  return groups > 1 ? (blockIdx.x % groups) * (gridDim.x / groups) + blockIdx.x / groups : blockIdx.x;
}

// ---- fp32: one thread per 4-channel, 16-byte vector ---------------------------
// Every lane of a wave takes the same path whatever its mask bytes (a lane
// with only local channels still loads and stores its T vectors), so no lane
// serialises the wave's loads behind a divergent branch.  In place, lanes with
// no synced channel leave at once, and mixed vectors write synced channels only.
template <int TC>  // TC = T known at compile time (1..16), or 0 for a runtime T
__global__ void __launch_bounds__(kReduceThreads)
pcr_reduce_f32_kernel(const float* Y, const uint8_t* __restrict__ mask, float* out,
                      int T_rt, uint32_t nvec, uint32_t hvec, long long mh, int inplace,
                       uint32_t groups) {
  const int T = TC > 0 ? TC : T_rt;
  const uint32_t v = reduce_block(groups) * kReduceThreads + threadIdx.x;
  if (v >= nvec) return;
  const int c = (int)(v % hvec) * 4;
  const long long base = (long long)v * 4;
  const uint32_t mk = *reinterpret_cast<const uint32_t*>(mask + c);
  const bool s0 = (mk & 0xffu) != 0, s1 = (mk & 0xff00u) != 0;
  const bool s2 = (mk & 0xff0000u) != 0, s3 = (mk & 0xff000000u) != 0;
  const bool all = s0 & s1 & s2 & s3;
  if (inplace && mk == 0u) return;
  if (TC > 0) {
    // All T vectors stay in registers: T loads in flight, then T stores.
    f32x4 y[TC > 0 ? TC : 1];
#pragma unroll
    for (int t = 0; t < (TC > 0 ? TC : 1); ++t)
      y[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + t * mh + base));
    f32x4 s = y[0];
#pragma unroll
    for (int t = 1; t < (TC > 0 ? TC : 1); ++t) s += y[t];
#pragma unroll
    for (int t = 0; t < (TC > 0 ? TC : 1); ++t) {
      float* o = out + t * mh + base;
      if (!inplace || all) {
        f32x4 w;
        w.x = s0 ? s.x : y[t].x;
        w.y = s1 ? s.y : y[t].y;
        w.z = s2 ? s.z : y[t].z;
        w.w = s3 ? s.w : y[t].w;
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(o));
      } else {  // in place, mixed vector: touch only the synced channels
        if (s0) o[0] = s.x;
        if (s1) o[1] = s.y;
        if (s2) o[2] = s.z;
        if (s3) o[3] = s.w;
      }
    }
  } else {
    // Runtime T: first pass sums, second pass writes (re-reading rank t's
    // vector for the local channels); both take the ranks eight at a time
    // with the group's loads in flight together.
    f32x4 s;
    for (int t0 = 0; t0 < T; t0 += 8) {
      f32x4 g[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + k < T) g[k] = *reinterpret_cast<const f32x4*>(Y + (t0 + k) * mh + base);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + k < T) s = t0 + k == 0 ? g[k] : s + g[k];
    }
    for (int t0 = 0; t0 < T; t0 += 8) {
      f32x4 g[8];
      if (!inplace || all)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (t0 + k < T) g[k] = *reinterpret_cast<const f32x4*>(Y + (t0 + k) * mh + base);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (t0 + k >= T) break;
        float* o = out + (t0 + k) * mh + base;
        if (!inplace || all) {
          f32x4 w;
          w.x = s0 ? s.x : g[k].x;
          w.y = s1 ? s.y : g[k].y;
          w.z = s2 ? s.z : g[k].z;
          w.w = s3 ? s.w : g[k].w;
          __builtin_nontemporal_store(w, reinterpret_cast<f32x4*>(o));
        } else {
          if (s0) o[0] = s.x;
          if (s1) o[1] = s.y;
          if (s2) o[2] = s.z;
          if (s3) o[3] = s.w;
        }
      }
    }
  }
}

// ---- fp32, T = 8, out of place: stores regrouped by rank --------------------
// The eight rank slices of Y and out lie M*H*4 bytes apart (256 MiB at
// M = 16384, H = 4096), so a thread's eight stores at one offset fall on the
// same HBM channels.  Here the 512 threads of a workgroup leave their eight
// output vectors in LDS and then wave t writes rank t's 8 KiB run of the
// block: the same values and loads as pcr_reduce_f32_kernel<8>, the stores
// in another order.
constexpr int kReduceRunThreads = 512;

__global__ void __launch_bounds__(kReduceRunThreads)
pcr_reduce_f32_runs8_kernel(const float* __restrict__ Y, const uint8_t* __restrict__ mask, float* __restrict__ out,
                            uint32_t nvec, uint32_t hvec, long long mh, uint32_t groups) {
  constexpr int TC = 8, NT = kReduceRunThreads;
  static_assert(NT / 64 == TC, "one wave per rank");
  __shared__ __attribute__((aligned(16))) f32x4 st[TC][NT];
  const uint32_t blk0 = reduce_block(groups) * NT;
  const uint32_t v = blk0 + threadIdx.x;
  if (v < nvec) {
    const int c = (int)(v % hvec) * 4;
    const long long base = (long long)v * 4;
    const uint32_t mk = *reinterpret_cast<const uint32_t*>(mask + c);
    const bool s0 = (mk & 0xffu) != 0, s1 = (mk & 0xff00u) != 0;
    const bool s2 = (mk & 0xff0000u) != 0, s3 = (mk & 0xff000000u) != 0;
    f32x4 y[TC];
#pragma unroll
    for (int t = 0; t < TC; ++t) y[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + t * mh + base));
    f32x4 s = y[0];
#pragma unroll
    for (int t = 1; t < TC; ++t) s += y[t];
#pragma unroll
    for (int t = 0; t < TC; ++t) {
      f32x4 w;
      w.x = s0 ? s.x : y[t].x;
      w.y = s1 ? s.y : y[t].y;
      w.z = s2 ? s.z : y[t].z;
      w.w = s3 ? s.w : y[t].w;
      st[t][threadIdx.x] = w;
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const int j = k * 64 + lane;
    if (blk0 + j < nvec)
      __builtin_nontemporal_store(st[t][j], reinterpret_cast<f32x4*>(out + t * mh + (long long)(blk0 + j) * 4));
  }
}

// ---- fp32 in, bf16 out: the second pass of the split forward ----------------
// out[t] = bf16 of the partial channel-reduce of the fp32 per-rank products
// Y[T,M,H]: on synced channels the ascending-rank fp32 sum starting from rank
// 0's value, elsewhere Y[t]; one thread per 4-channel vector, T 16-byte loads
// and T 8-byte stores.  With ks > 1 the products come in ks contraction
// slices, Y[q][t] at Y + q * sstride + t * mh, and rank t's value is their
// fp32 sum in slice order.  skip_local (H a multiple of 64): 64-channel
// groups with no synced channel were written to out by the first pass (Y
// holds nothing there); the 16 consecutive threads that cover such a group
// find that out together and leave.
template <int TC>  // TC = T known at compile time (1..16), or 0 for a runtime T
__global__ void __launch_bounds__(kReduceThreads)
pcr_reduce_f32_bf16_kernel(const float* __restrict__ Y, const uint8_t* __restrict__ mask, uint16_t* __restrict__ out,
                           int T_rt, uint32_t nvec, uint32_t hvec, long long mh, uint32_t groups, int ks,
                           long long sstride, int skip_local) {
  const int T = TC > 0 ? TC : T_rt;
  constexpr int NR = TC > 0 ? TC : 1;  // ranks kept in registers
  const uint32_t v = reduce_block(groups) * kReduceThreads + threadIdx.x;
  if (v >= nvec) return;
  const int c = (int)(v % hvec) * 4;
  const long long base = (long long)v * 4;
  const uint32_t mk = *reinterpret_cast<const uint32_t*>(mask + c);
  if (skip_local) {
    // nvec and the 64-channel groups are multiples of 16 threads, so the 16
    // lanes of a group are all here
    uint32_t any = mk;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) any |= __shfl_xor(any, o, 16);
    if (any == 0u) return;
  }
  const bool s0 = (mk & 0xffu) != 0, s1 = (mk & 0xff00u) != 0;
  const bool s2 = (mk & 0xff0000u) != 0, s3 = (mk & 0xff000000u) != 0;
  // Runtime T: a rank's product (its slices in slice order) is read twice,
  // for the sum and for the output, with plain loads so the second read
  // finds the lines in cache; ranks go eight at a time, the group's loads in
  // flight together.
  auto rank_group = [&](int t0, f32x4 (&g)[8]) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (t0 + k < T) g[k] = *reinterpret_cast<const f32x4*>(Y + (t0 + k) * mh + base);
    for (int q = 1; q < ks; ++q)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + k < T) g[k] += *reinterpret_cast<const f32x4*>(Y + q * sstride + (t0 + k) * mh + base);
  };
  f32x4 y[NR];
  f32x4 s;
  if (TC > 0) {
#pragma unroll
    for (int t = 0; t < NR; ++t) y[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + t * mh + base));
    for (int q = 1; q < ks; ++q)
#pragma unroll
      for (int t = 0; t < NR; ++t)
        y[t] += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Y + q * sstride + t * mh + base));
    s = y[0];
#pragma unroll
    for (int t = 1; t < NR; ++t) s += y[t];
  } else {
    for (int t0 = 0; t0 < T; t0 += 8) {
      f32x4 g[8];
      rank_group(t0, g);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + k < T) s = t0 + k == 0 ? g[k] : s + g[k];
    }
  }
  auto put = [&](int t, f32x4 yt) {
    u32x2 o;
    o[0] = pack_bf16x2(s0 ? s.x : yt.x, s1 ? s.y : yt.y);
    o[1] = pack_bf16x2(s2 ? s.z : yt.z, s3 ? s.w : yt.w);
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(out + t * mh + base));
  };
  if constexpr (TC > 0) {
#pragma unroll
    for (int t = 0; t < NR; ++t) put(t, y[t]);
  } else {
    for (int t0 = 0; t0 < T; t0 += 8) {
      f32x4 g[8];
      rank_group(t0, g);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + k < T) put(t0 + k, g[k]);
    }
  }
}

// ---- classes of 256-channel tiles, for the backward's reduced gradient -------
// With a contiguous sync set most tiles of channels are wholly synced or
// wholly local.  Then the backward's G needs no per-rank copy there: a wholly
// local tile of G_t is dZ_t itself, and a wholly synced one is the same sum
// for every rank, stored once (in rank 0's slot).  tbits[0] has bit i set when
// every channel of tile i (channels 256 i .. 256 i + 255, or up to H) is
// synced, tbits[1] when none is; tiles up to kMaxClassTiles (H <= 16384).
constexpr int kClassCols = 256;
constexpr int kMaxClassTiles = 64;

__device__ __forceinline__ bool no_zero_byte(uint32_t w) { return ((w - 0x01010101u) & ~w & 0x80808080u) == 0u; }

__global__ void __launch_bounds__(64) pcr_tile_class_kernel(const uint8_t* __restrict__ mask, int H,
                                                            unsigned long long* tbits) {
  const int c0 = threadIdx.x * kClassCols;  // one tile per lane
  bool all = c0 < H, none = c0 < H;
  // All of the lane's 8-byte mask words are loaded at once (no early exit);
  // words past H count as neither.
#pragma unroll
  for (int i = 0; i < kClassCols / 8; ++i) {  // H % 8 == 0
    const int c = c0 + 8 * i;
    if (c < H) {
      const u32x2 mk = *reinterpret_cast<const u32x2*>(mask + c);
      all &= no_zero_byte(mk[0]) & no_zero_byte(mk[1]);
      none &= (mk[0] | mk[1]) == 0u;
    }
  }
  const unsigned long long sb = __ballot(all), lb = __ballot(none);
  if (threadIdx.x == 0) {
    tbits[0] = sb;
    tbits[1] = lb;
  }
}

// ---- bf16: one thread per 8-channel, 16-byte vector ---------------------------

__device__ __forceinline__ void bf16x8_to_f32(const u32x4 v, float f[8]) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    f[2 * d] = bf16_lo(v[d]);
    f[2 * d + 1] = bf16_hi(v[d]);
  }
}

// 0xffff per synced bf16 lane of an 8-channel vector, from 8 mask bytes.
__device__ __forceinline__ u32x4 expand_mask8(uint32_t lo, uint32_t hi) {
  u32x4 r;
  r[0] = ((lo & 0xffu) ? 0xffffu : 0u) | ((lo & 0xff00u) ? 0xffff0000u : 0u);
  r[1] = ((lo & 0xff0000u) ? 0xffffu : 0u) | ((lo & 0xff000000u) ? 0xffff0000u : 0u);
  r[2] = ((hi & 0xffu) ? 0xffffu : 0u) | ((hi & 0xff00u) ? 0xffff0000u : 0u);
  r[3] = ((hi & 0xff0000u) ? 0xffffu : 0u) | ((hi & 0xff000000u) ? 0xffff0000u : 0u);
  return r;
}

template <int TC>  // TC = T known at compile time (1..16), or 0 for a runtime T
__global__ void __launch_bounds__(kReduceThreads)
pcr_reduce_bf16_kernel(const uint16_t* Y, const uint8_t* __restrict__ mask, uint16_t* out,
                       int T_rt, uint32_t nvec, uint32_t hvec, long long mh, int inplace,
                       uint32_t groups, const unsigned long long* __restrict__ tbits) {
  const int T = TC > 0 ? TC : T_rt;
  constexpr int NR = TC > 0 ? TC : 1;  // ranks kept in registers
  const uint32_t v = reduce_block(groups) * kReduceThreads + threadIdx.x;
  if (v >= nvec) return;
  const int c = (int)(v % hvec) * 8;
  const long long base = (long long)v * 8;
  // The backward's G with tile classes (tbits != nullptr, never in place):
  // nothing to write for a wholly local tile, one copy (rank 0's slot) of
  // the sum for a wholly synced one.
  int ranks_out = T;
  if (tbits != nullptr) {
    const int tile = c / kClassCols;
    if ((tbits[1] >> tile) & 1ull) return;
    if ((tbits[0] >> tile) & 1ull) ranks_out = 1;
  }
  const u32x2 mk = *reinterpret_cast<const u32x2*>(mask + c);
  if (inplace && (mk[0] | mk[1]) == 0u) return;
  const u32x4 sel = expand_mask8(mk[0], mk[1]);
  const bool all = (sel[0] & sel[1] & sel[2] & sel[3]) == 0xffffffffu;
  u32x4 y[NR];
  float s[8];
  if (TC > 0) {
#pragma unroll
    for (int t = 0; t < NR; ++t) y[t] = ld16(Y + t * mh + base);
    bf16x8_to_f32(y[0], s);
#pragma unroll
    for (int t = 1; t < NR; ++t) {
      float f[8];
      bf16x8_to_f32(y[t], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += f[e];
    }
  } else {
    // Runtime T: ranks eight at a time, the group's loads in flight together.
    for (int t0 = 0; t0 < T; t0 += 8) {
      u32x4 g[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + k < T) g[k] = ld16(Y + (t0 + k) * mh + base);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + k < T) {
          float f[8];
          bf16x8_to_f32(g[k], f);
#pragma unroll
          for (int e = 0; e < 8; ++e) s[e] = t0 + k == 0 ? f[e] : s[e] + f[e];
        }
    }
  }
  u32x4 sv;
#pragma unroll
  for (int d = 0; d < 4; ++d) sv[d] = pack_bf16x2(s[2 * d], s[2 * d + 1]);
  auto put = [&](int t, u32x4 yt) {
    uint16_t* o = out + t * mh + base;
    if (!inplace || all) {
      st16_nt(o, (sv & sel) | (yt & ~sel));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if ((sel[e >> 1] >> (16 * (e & 1))) & 1u) o[e] = (uint16_t)(sv[e >> 1] >> (16 * (e & 1)));
    }
  };
  if constexpr (TC > 0) {
#pragma unroll
    for (int t = 0; t < NR; ++t)
      if (t < ranks_out) put(t, y[t]);
  } else {
    // Every load of a group goes out before its first store (each element is
    // still read before it is written, by the same thread, in place too).
    for (int t0 = 0; t0 < ranks_out; t0 += 8) {
      u32x4 g[8];
      if (!inplace || all)
#pragma unroll
        for (int k = 0; k < 8; ++k)
          if (t0 + k < ranks_out) g[k] = ld16(Y + (t0 + k) * mh + base);
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + k < ranks_out) put(t0 + k, g[k]);
    }
  }
}

// ---- bf16, T = 8, out of place: stores regrouped by rank --------------------
// As pcr_reduce_f32_runs8_kernel for the bf16 reduce (the backward's G with
// tile classes: a vector writes no rank, rank 0 only, or all eight).
__global__ void __launch_bounds__(kReduceRunThreads)
pcr_reduce_bf16_runs8_kernel(const uint16_t* __restrict__ Y, const uint8_t* __restrict__ mask,
                             uint16_t* __restrict__ out, uint32_t nvec, uint32_t hvec, long long mh, uint32_t groups,
                             const unsigned long long* __restrict__ tbits) {
  constexpr int TC = 8, NT = kReduceRunThreads;
  __shared__ __attribute__((aligned(16))) u32x4 st[TC][NT];
  __shared__ uint8_t nout[NT];
  const uint32_t blk0 = reduce_block(groups) * NT;
  const uint32_t v = blk0 + threadIdx.x;
  int ranks_out = 0;
  if (v < nvec) {
    const int c = (int)(v % hvec) * 8;
    const long long base = (long long)v * 8;
    ranks_out = TC;
    if (tbits != nullptr) {
      const int tile = c / kClassCols;
      if ((tbits[1] >> tile) & 1ull) ranks_out = 0;
      else if ((tbits[0] >> tile) & 1ull) ranks_out = 1;
    }
    if (ranks_out > 0) {
      const u32x2 mk = *reinterpret_cast<const u32x2*>(mask + c);
      const u32x4 sel = expand_mask8(mk[0], mk[1]);
      u32x4 y[TC];
#pragma unroll
      for (int t = 0; t < TC; ++t) y[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Y + t * mh + base));
      float s[8];
      bf16x8_to_f32(y[0], s);
#pragma unroll
      for (int t = 1; t < TC; ++t) {
        float f[8];
        bf16x8_to_f32(y[t], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += f[e];
      }
      u32x4 sv;
#pragma unroll
      for (int d = 0; d < 4; ++d) sv[d] = pack_bf16x2(s[2 * d], s[2 * d + 1]);
#pragma unroll
      for (int t = 0; t < TC; ++t) st[t][threadIdx.x] = (sv & sel) | (y[t] & ~sel);
    }
  }
  nout[threadIdx.x] = (uint8_t)ranks_out;
  __syncthreads();
  const int lane = threadIdx.x & 63, t = threadIdx.x >> 6;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) {
    const int j = k * 64 + lane;
    if (blk0 + j < nvec && t < nout[j]) st16_nt(out + t * mh + (long long)(blk0 + j) * 8, st[t][j]);
  }
}

// ---- bf16, T = 16, out of place: stores regrouped by rank -------------------
// As pcr_reduce_bf16_runs8_kernel with sixteen ranks: each wave writes two
// ranks' 8 KiB runs of the block (128 KiB of LDS).
__global__ void __launch_bounds__(kReduceRunThreads)
pcr_reduce_bf16_runs16_kernel(const uint16_t* __restrict__ Y, const uint8_t* __restrict__ mask,
                              uint16_t* __restrict__ out, uint32_t nvec, uint32_t hvec, long long mh, uint32_t groups,
                              const unsigned long long* __restrict__ tbits) {
  constexpr int TC = 16, NT = kReduceRunThreads;
  __shared__ __attribute__((aligned(16))) u32x4 st[TC][NT];
  __shared__ uint8_t nout[NT];
  const uint32_t blk0 = reduce_block(groups) * NT;
  const uint32_t v = blk0 + threadIdx.x;
  int ranks_out = 0;
  if (v < nvec) {
    const int c = (int)(v % hvec) * 8;
    const long long base = (long long)v * 8;
    ranks_out = TC;
    if (tbits != nullptr) {
      const int tile = c / kClassCols;
      if ((tbits[1] >> tile) & 1ull) ranks_out = 0;
      else if ((tbits[0] >> tile) & 1ull) ranks_out = 1;
    }
    if (ranks_out > 0) {
      const u32x2 mk = *reinterpret_cast<const u32x2*>(mask + c);
      const u32x4 sel = expand_mask8(mk[0], mk[1]);
      u32x4 y[TC];
#pragma unroll
      for (int t = 0; t < TC; ++t) y[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Y + t * mh + base));
      float s[8];
      bf16x8_to_f32(y[0], s);
#pragma unroll
      for (int t = 1; t < TC; ++t) {
        float f[8];
        bf16x8_to_f32(y[t], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] += f[e];
      }
      u32x4 sv;
#pragma unroll
      for (int d = 0; d < 4; ++d) sv[d] = pack_bf16x2(s[2 * d], s[2 * d + 1]);
#pragma unroll
      for (int t = 0; t < TC; ++t) st[t][threadIdx.x] = (sv & sel) | (y[t] & ~sel);
    }
  }
  nout[threadIdx.x] = (uint8_t)ranks_out;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int rr = 0; rr < 2; ++rr) {
    const int t = 2 * wave + rr;
#pragma unroll
    for (int k = 0; k < NT / 64; ++k) {
      const int j = k * 64 + lane;
      if (blk0 + j < nvec && t < nout[j]) st16_nt(out + t * mh + (long long)(blk0 + j) * 8, st[t][j]);
    }
  }
}

// Small fill kernel (used instead of a runtime memset so the call sequence can
// be captured in a graph).
__global__ void fill_u32_kernel(uint32_t* p, long long n, uint32_t v) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace caat
