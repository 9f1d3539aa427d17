// The three MFMA GEMMs of the row-parallel layer with partial channel-reduce.
//
// Layer (CAAT-Net paper, Introduction): T tensor-parallel ranks each hold
// X_t[M,Kr] and W_t[Kr,H]; the row-parallel product Y_t = X_t W_t is followed
// by a reduce over only the sync-set channels S; other channels stay local.
//
//   forward   Z_t[:,c] = sum_u Y_u[:,c]  (c in S),   Y_t[:,c]  (c not in S)
//   backward  G_t = the same reduce applied to dZ;  dX_t = G_t W_t^T;  dW_t = X_t^T G_t
#pragma once

#include "gemm_core.hpp"
#include "reduce_kernels.hpp"

namespace caat {

// ============================================================================
// Forward: one workgroup per (m-tile, n-tile) walks the contraction of all T
// ranks in rank order.  Synced columns keep accumulating across the rank
// boundaries, so their fp32 accumulator ends as the sum over ranks (ascending
// t), formed once and written to every rank: bit-identical synced channels.
// Local columns are written to out[t] at the end of rank t and restarted from
// zero.  No fp32 partial ever leaves the registers.
// ============================================================================
template <int BM, int BN>
__global__ void __launch_bounds__(kGemmThreads, 1)
rowpar_pcr_fwd_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                      const uint8_t* __restrict__ mask, uint16_t* __restrict__ out,
                      int T, int M, int Kr, int H, int tiles_m, int tiles_n) {
  using S = TileShape<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int nk = (Kr + kBK - 1) / kBK;
  const long long MK = (long long)M * Kr, KH = (long long)Kr * H, MH = (long long)M * H;

  int col[S::WJ];
  bool cok[S::WJ], syn[S::WJ];
#pragma unroll
  for (int j = 0; j < S::WJ; ++j) {
    col[j] = n0 + wn * S::WN + j * 32 + (lane & 31);
    cok[j] = col[j] < H;
    syn[j] = cok[j] && mask[col[j]] != 0;
  }

  f32x16 acc[S::WI][S::WJ];
#pragma unroll
  for (int i = 0; i < S::WI; ++i)
#pragma unroll
    for (int j = 0; j < S::WJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  KContLoader<BM> la;
  MNContLoader<BN> lb;
  const u32x4 zero = {0u, 0u, 0u, 0u};

  auto load = [&](int c) {
    const int t = c / nk;
    const int k0 = (c - t * nk) * kBK;
    const uint16_t* Xt = X + t * MK;
    const uint16_t* Wt = W + t * KH;
    la.load(
        [&](int r, int k) -> u32x4 {
          const int row = min(m0 + r, M - 1);
          const u32x4 v = ld16(Xt + (uint32_t)(row * Kr + min(k0 + k, Kr - 8)));
          return (k0 + k < Kr) ? v : zero;
        },
        tid);
    lb.load(
        [&](int kk, int n) -> u32x4 {
          const int cc = min(n0 + n, H - 8);
          const u32x4 v = ld16(Wt + (uint32_t)(min(k0 + kk, Kr - 1) * H + cc));
          return (k0 + kk < Kr) ? v : zero;
        },
        tid);
  };
  auto store = [&](uint16_t* a, uint16_t* b) {
    la.store(a, tid);
    lb.store(b, tid);
  };
  // Straight-line epilogues (no divergent branches around the accumulators):
  // stores are predicated per lane, local accumulators are cleared with a mask.
  uint32_t keep[S::WJ];  // all ones for synced columns, zero for local ones
#pragma unroll
  for (int j = 0; j < S::WJ; ++j) keep[j] = syn[j] ? 0xffffffffu : 0u;
  auto rank_end = [&](int t) {
    // Opaque per-call copies of the lane's first row and column: the store
    // addresses derived from them cannot be hoisted out of the chunk loop
    // (256 hoisted addresses would not fit in registers).
    int rbase = m0 + wm * S::WM + (lane >> 5) * 4;
    int cbase = n0 + wn * S::WN + (lane & 31);
    asm volatile("" : "+v"(rbase), "+v"(cbase));
    uint16_t* ot = out + t * MH;
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int j = 0; j < S::WJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + (e >> 2) * 8 + (e & 3);
          const float v = acc[i][j][e];
          if (!syn[j] && cok[j] && row < M) ot[(long long)row * H + cbase + j * 32] = f32_to_bf16(v);
          acc[i][j][e] = __uint_as_float(__float_as_uint(v) & keep[j]);
        }
  };
  gemm_mainloop_ranks<BM, BN>(smem, T, nk, load, store, rank_end, acc);

  // Last rank: its local channels, and the synced channels for every rank.
  for (int u = 0; u < T; ++u) {
    int rbase = m0 + wm * S::WM + (lane >> 5) * 4;
    int cbase = n0 + wn * S::WN + (lane & 31);
    asm volatile("" : "+v"(rbase), "+v"(cbase));
    const bool last = u == T - 1;
    uint16_t* ou = out + u * MH;
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int j = 0; j < S::WJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = rbase + i * 32 + (e >> 2) * 8 + (e & 3);
          if ((syn[j] || last) && cok[j] && row < M)
            ou[(long long)row * H + cbase + j * 32] = f32_to_bf16(acc[i][j][e]);
        }
  }
}

// ============================================================================
// Backward, input gradient: dX_t[m,k] = sum_c G_t[m,c] W_t[k,c].
// A = G_t (rows m, contraction c contiguous), selected per channel between the
// synced sum Gs and the rank's own dZ_t; B = W_t read as [k][c] (c contiguous).
// ============================================================================
template <int BM, int BN>
__global__ void __launch_bounds__(kGemmThreads, 1)
pcr_bwd_dx_kernel(const uint16_t* __restrict__ dZ, const uint16_t* __restrict__ Gs,
                  const uint16_t* __restrict__ W, const uint8_t* __restrict__ mask,
                  uint16_t* __restrict__ dX, int T, int M, int Kr, int H, int tiles_m, int tiles_n) {
  using S = TileShape<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int per_rank = tiles_m * tiles_n;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int t = lin / per_rank;
  int tm, tn;
  tile_coords(lin - t * per_rank, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const long long MH = (long long)M * H, KH = (long long)Kr * H;
  const uint16_t* dZt = dZ + t * MH;
  const uint16_t* Wt = W + t * KH;

  f32x16 acc[S::WI][S::WJ];
#pragma unroll
  for (int i = 0; i < S::WI; ++i)
#pragma unroll
    for (int j = 0; j < S::WJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  KContLoader<BM> la;
  KContLoader<BN> lb;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load = [&](int c) {
    const int k0 = c * kBK;
    la.load(
        [&](int r, int k) -> u32x4 {
          const int row = min(m0 + r, M - 1);
          const int ch = k0 + k;
          if (ch >= H) return zero;
          const u32x2 mk = *reinterpret_cast<const u32x2*>(mask + ch);
          const long long off = (long long)row * H + ch;
          if ((mk[0] | mk[1]) == 0u) return ld16(dZt + off);
          const u32x4 sel = expand_mask8(mk[0], mk[1]);
          const u32x4 gs = ld16(Gs + off);
          if ((sel[0] & sel[1] & sel[2] & sel[3]) == 0xffffffffu) return gs;
          return (gs & sel) | (ld16(dZt + off) & ~sel);
        },
        tid);
    lb.load(
        [&](int r, int k) -> u32x4 {
          const int row = min(n0 + r, Kr - 1);
          return (k0 + k < H) ? ld16(Wt + (long long)row * H + k0 + k) : zero;
        },
        tid);
  };
  auto store = [&](uint16_t* a, uint16_t* b) {
    la.store(a, tid);
    lb.store(b, tid);
  };
  gemm_mainloop<BM, BN>(smem, (H + kBK - 1) / kBK, load, store, [](int) {}, acc);

  uint16_t* dXt = dX + (long long)t * M * Kr;
#pragma unroll
  for (int j = 0; j < S::WJ; ++j) {
    const int cc = n0 + wn * S::WN + j * 32 + (lane & 31);
    if (cc >= Kr) continue;
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * S::WM + i * 32 + acc_row(e, lane);
        if (row < M) dXt[(long long)row * Kr + cc] = f32_to_bf16(acc[i][j][e]);
      }
  }
}

// ============================================================================
// Backward, weight gradient: dW_t[k,c] = sum_m X_t[m,k] G_t[m,c].
// The contraction runs over tokens m, which is the strided index of both
// operands, so both are loaded as 8x8 blocks and transposed in registers.
// ============================================================================
template <int BM, int BN>
__global__ void __launch_bounds__(kGemmThreads, 1)
pcr_bwd_dw_kernel(const uint16_t* __restrict__ dZ, const uint16_t* __restrict__ Gs,
                  const uint16_t* __restrict__ X, const uint8_t* __restrict__ mask,
                  uint16_t* __restrict__ dW, int T, int M, int Kr, int H, int tiles_m, int tiles_n) {
  using S = TileShape<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int per_rank = tiles_m * tiles_n;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int t = lin / per_rank;
  int tm, tn;
  tile_coords(lin - t * per_rank, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;  // m0 over Kr (rows of dW), n0 over H
  const long long MH = (long long)M * H, MK = (long long)M * Kr;
  const uint16_t* dZt = dZ + t * MH;
  const uint16_t* Xt = X + t * MK;

  f32x16 acc[S::WI][S::WJ];
#pragma unroll
  for (int i = 0; i < S::WI; ++i)
#pragma unroll
    for (int j = 0; j < S::WJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  MNContLoader<BM> la;
  MNContLoader<BN> lb;
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load = [&](int c) {
    const int k0 = c * kBK;  // token index
    la.load(
        [&](int kk, int r) -> u32x4 {
          const int m = k0 + kk;
          const int kcol = min(m0 + r, Kr - 8);
          return (m < M) ? ld16(Xt + (long long)m * Kr + kcol) : zero;
        },
        tid);
    lb.load(
        [&](int kk, int r) -> u32x4 {
          const int m = k0 + kk;
          const int ch = min(n0 + r, H - 8);
          if (m >= M) return zero;
          const u32x2 mk = *reinterpret_cast<const u32x2*>(mask + ch);
          const long long off = (long long)m * H + ch;
          if ((mk[0] | mk[1]) == 0u) return ld16(dZt + off);
          const u32x4 sel = expand_mask8(mk[0], mk[1]);
          const u32x4 gs = ld16(Gs + off);
          if ((sel[0] & sel[1] & sel[2] & sel[3]) == 0xffffffffu) return gs;
          return (gs & sel) | (ld16(dZt + off) & ~sel);
        },
        tid);
  };
  auto store = [&](uint16_t* a, uint16_t* b) {
    la.store(a, tid);
    lb.store(b, tid);
  };
  gemm_mainloop<BM, BN>(smem, (M + kBK - 1) / kBK, load, store, [](int) {}, acc);

  uint16_t* dWt = dW + (long long)t * Kr * H;
#pragma unroll
  for (int j = 0; j < S::WJ; ++j) {
    const int cc = n0 + wn * S::WN + j * 32 + (lane & 31);
    if (cc >= H) continue;
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * S::WM + i * 32 + acc_row(e, lane);
        if (row < Kr) dWt[(long long)row * H + cc] = f32_to_bf16(acc[i][j][e]);
      }
  }
}

}  // namespace caat
