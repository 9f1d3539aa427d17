// The three MFMA GEMMs of the row-parallel layer with partial channel-reduce.
//
// Layer (CAAT-Net paper, Introduction): T tensor-parallel ranks each hold
// X_t[M,Kr] and W_t[Kr,H]; the row-parallel product Y_t = X_t W_t is followed
// by a reduce over only the sync-set channels S; other channels stay local.
//
//   forward   Z_t[:,c] = sum_u Y_u[:,c]  (c in S),   Y_t[:,c]  (c not in S)
//   backward  G_t = the same reduce applied to dZ;  dX_t = G_t W_t^T;  dW_t = X_t^T G_t
//
// Every GEMM computes the transpose of its output tile (the MFMA row index is
// the output's contiguous index), so each lane holds runs of 4 consecutive
// output elements and writes them with one 8-byte store.
#pragma once

#include "gemm_core.hpp"
#include "reduce_kernels.hpp"

namespace caat {

// Opaque copy of a value: addresses derived from it are recomputed where they
// are used instead of being hoisted (and kept live) across the main loop.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// 4 accumulator values (registers 4q..4q+3 of a block) as 4 packed bf16.
__device__ __forceinline__ u32x2 pack4(const f32x16& a, int q) {
  u32x2 r;
  r[0] = pack_bf16x2(a[4 * q], a[4 * q + 1]);
  r[1] = pack_bf16x2(a[4 * q + 2], a[4 * q + 3]);
  return r;
}
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }


// ============================================================================
// Forward.  One workgroup per (channel tile, token tile) walks the contraction
// of all T ranks in rank order.  Synced channels keep accumulating across the
// rank boundaries, so their fp32 accumulator ends as the sum over ranks
// (ascending t), formed once and written to every rank: bit-identical synced
// channels.  At the end of rank t its 4-channel groups are written to out[t]
// (the synced lanes of a group hold a partial sum there and are rewritten at
// the end) and the local accumulators restart from zero.  At the end, rank
// T-1 gets whole groups; every other rank gets its groups read back, merged
// with the synced channels, and written again.
// A = W_t^T (channels x k, W is [k][c]: MNCONT); B = X_t (tokens x k: KCONT).
// ============================================================================
template <int BM, int BN>
__global__ void __launch_bounds__(kGemmThreads, 1)
rowpar_pcr_fwd_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                      const uint8_t* __restrict__ mask, uint16_t* __restrict__ out,
                      int T, int M, int Kr, int H, int tiles_m, int tiles_n) {
  using S = TileShape<BM, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int c0 = tm * BM, m0 = tn * BN;  // channel tile, token tile
  const int nk = (Kr + kBK - 1) / kBK;
  const int kv_last = Kr - (nk - 1) * kBK;  // valid k in a rank's last chunk
  const int nchunks = T * nk;
  const long long MK = (long long)M * Kr, KH = (long long)Kr * H, MH = (long long)M * H;

  // Per lane: channel group q of block i starts at chan(i, q); keep[i] has bit
  // e set when accumulator register e of block i is a synced channel.
  const int cl = c0 + wm * S::WM + (lane >> 5) * 4;
  uint32_t keepbits[S::WI];
#pragma unroll
  for (int i = 0; i < S::WI; ++i) {
    uint32_t kb = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = cl + i * 32 + q * 8;
      const uint32_t m4 = ch < H ? *reinterpret_cast<const uint32_t*>(mask + ch) : 0u;
#pragma unroll
      for (int r = 0; r < 4; ++r) kb |= ((m4 >> (8 * r)) & 0xffu) ? (1u << (4 * q + r)) : 0u;
    }
    keepbits[i] = kb;
  }

  f32x16 acc[S::WI][S::WJ];
  zero_acc<BM, BN>(acc);

  auto issue = [&](int c) {
    const int t = c / nk;
    const int k0 = (c - t * nk) * kBK;
    uint16_t* buf = smem + (c & 1) * S::BUF;
    const MnDma<BM> da(W + t * KH, (uint32_t)(KH * 2), H, lane, wave);
    const KcDma db(X + t * MK, (uint32_t)(MK * 2), Kr, lane);
    da.load(H, c0, k0, buf, wave);
    db.load<BN>(Kr, m0, k0, buf + BM * kBK, wave);
  };

  issue(0);
  for (int t = 0; t < T; ++t) {
    for (int kc = 0; kc < nk; ++kc) {
      const int c = t * nk + kc;
      uint16_t* As = smem + (c & 1) * S::BUF;
      uint16_t* Bs = As + BM * kBK;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kc == nk - 1 && kv_last < kBK) {  // W's rows past Kr arrived as zeros
        zero_kcont_tail<BN>(Bs, kv_last, tid);
        __syncthreads();
      }
      if (c + 1 < nchunks) issue(c + 1);
      mma_chunk<BM, BN>([&](int ks, int i) { return frag_mncont<BM>(As, wm * S::WM + i * 32, ks, lane); },
                        [&](int ks, int j) { return frag_kcont(Bs, wn * S::WN + j * 32, ks, lane); }, acc);
    }
    if (t + 1 < T) {
      // End of rank t: write its groups, then restart the local channels.
      const int chb = opaque(cl);
      const int tok = opaque(m0 + wn * S::WN + (lane & 31));
      uint16_t* ot = out + t * MH;
#pragma unroll
      for (int i = 0; i < S::WI; ++i) {
        const uint32_t kb = (uint32_t)opaque((int)keepbits[i]);
#pragma unroll
        for (int j = 0; j < S::WJ; ++j) {
          const int m = tok + j * 32;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ch = chb + i * 32 + q * 8;
            if (m < M && ch < H) st8(ot + (long long)m * H + ch, pack4(acc[i][j], q));
          }
#pragma unroll
          for (int e = 0; e < 16; ++e) {  // all ones where register e is a synced channel
            const uint32_t keep = (uint32_t)((int)(kb << (31 - e)) >> 31);
            acc[i][j][e] = __uint_as_float(__float_as_uint(acc[i][j][e]) & keep);
          }
        }
      }
    }
  }

  // Rank T-1: whole groups.  Ranks t < T-1: merge the synced channels into the
  // groups written at the end of rank t (by this same lane): all of a rank's
  // groups are read first, then merged and written.
  for (int u = T - 1; u >= 0; --u) {
    const int chb = opaque(cl);
    const int tok = opaque(m0 + wn * S::WN + (lane & 31));
    uint16_t* ou = out + u * MH;
    if (u == T - 1) {
#pragma unroll
      for (int i = 0; i < S::WI; ++i)
#pragma unroll
        for (int j = 0; j < S::WJ; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int ch = chb + i * 32 + q * 8, m = tok + j * 32;
            if (m < M && ch < H) st8(ou + (long long)m * H + ch, pack4(acc[i][j], q));
          }
      continue;
    }
    u32x2 old[S::WI][S::WJ][4];
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int j = 0; j < S::WJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = min(chb + i * 32 + q * 8, H - 4), m = min(tok + j * 32, M - 1);
          old[i][j][q] = ld8(ou + (long long)m * H + ch);
        }
#pragma unroll
    for (int i = 0; i < S::WI; ++i) {
      const uint32_t kb = (uint32_t)opaque((int)keepbits[i]);
#pragma unroll
      for (int j = 0; j < S::WJ; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ch = chb + i * 32 + q * 8, m = tok + j * 32;
          u32x2 sel;  // 0xffff per synced bf16 lane of the group
          sel[0] = (((kb >> (4 * q)) & 1u) ? 0xffffu : 0u) | (((kb >> (4 * q + 1)) & 1u) ? 0xffff0000u : 0u);
          sel[1] = (((kb >> (4 * q + 2)) & 1u) ? 0xffffu : 0u) | (((kb >> (4 * q + 3)) & 1u) ? 0xffff0000u : 0u);
          if (m < M && ch < H && ((kb >> (4 * q)) & 0xfu) != 0u)
            st8(ou + (long long)m * H + ch, (pack4(acc[i][j], q) & sel) | (old[i][j][q] & ~sel));
        }
    }
  }
}

// Rank t's reduced gradient, 8 channels: Gs where the mask is set, dZ_t elsewhere.
__device__ __forceinline__ u32x4 select8(u32x4 gs, u32x4 dz, u32x4 sel) { return (gs & sel) | (dz & ~sel); }

// ============================================================================
// Backward, input gradient, computed as dX_t^T[k,m] = sum_c W_t[k,c] G_t[m,c].
// A = W_t (rows k, contraction c contiguous: KCONT, copied directly);
// B = G_t (rows m: KCONT, staged through registers for the select).
// ============================================================================
template <int BM, int BN>
__global__ void __launch_bounds__(kGemmThreads, 1)
pcr_bwd_dx_kernel(const uint16_t* __restrict__ dZ, const uint16_t* __restrict__ Gs,
                  const uint16_t* __restrict__ W, const uint8_t* __restrict__ mask,
                  uint16_t* __restrict__ dX, int T, int M, int Kr, int H, int tiles_m, int tiles_n) {
  using S = TileShape<BM, BN>;
  constexpr int NV = BN * 8 / kGemmThreads;  // staged 16-byte vectors per thread
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int per_rank = tiles_m * tiles_n;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int t = lin / per_rank;
  int tm, tn;
  tile_coords(lin - t * per_rank, tiles_m, tiles_n, tm, tn);
  const int k0r = tm * BM, m0 = tn * BN;  // rows of W_t (dX columns), tokens
  const long long MH = (long long)M * H, KH = (long long)Kr * H;
  const uint16_t* dZt = dZ + t * MH;
  const uint16_t* Wt = W + t * KH;
  const int nk = (H + kBK - 1) / kBK;
  const int kv_last = H - (nk - 1) * kBK;

  f32x16 acc[S::WI][S::WJ];
  zero_acc<BM, BN>(acc);

  // Staged B: this thread always owns 16-byte chunk (tid & 7) of its token rows.
  const int my_chunk = tid & 7;
  u32x4 vz[NV], vg[NV];
  u32x4 sel;
  auto load_b = [&](int c) {
    const int ch = min(c * kBK + my_chunk * 8, H - 8);
    const u32x2 mk = *reinterpret_cast<const u32x2*>(mask + ch);
    sel = expand_mask8(mk[0], mk[1]);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int row = min(m0 + ((tid + i * kGemmThreads) >> 3), M - 1);
      const uint32_t off = (uint32_t)(row * H + ch);
      vz[i] = ld16(dZt + off);
      vg[i] = ld16(Gs + off);
    }
  };
  auto store_b = [&](int c, uint16_t* Bs) {
    const bool inside = c * kBK + my_chunk * 8 < H;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int row = (tid + i * kGemmThreads) >> 3;
      st16(Bs + kc_off(row, my_chunk), inside ? select8(vg[i], vz[i], sel) : z);
    }
  };
  const KcDma da(Wt, (uint32_t)(KH * 2), H, lane);
  auto issue_a = [&](int c) { da.load<BM>(H, k0r, c * kBK, smem + (c & 1) * S::BUF, wave); };

  load_b(0);
  issue_a(0);
  store_b(0, smem + BM * kBK);
  for (int c = 0; c < nk; ++c) {
    uint16_t* As = smem + (c & 1) * S::BUF;
    uint16_t* Bs = As + BM * kBK;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c == nk - 1 && kv_last < kBK) {
      zero_kcont_tail<BM>(As, kv_last, tid);
      __syncthreads();
    }
    const bool more = c + 1 < nk;
    if (more) {
      load_b(c + 1);
      issue_a(c + 1);
    }
    mma_chunk<BM, BN>([&](int ks, int i) { return frag_kcont(As, wm * S::WM + i * 32, ks, lane); },
                      [&](int ks, int j) { return frag_kcont(Bs, wn * S::WN + j * 32, ks, lane); }, acc);
    if (more) store_b(c + 1, smem + ((c + 1) & 1) * S::BUF + BM * kBK);
  }

  uint16_t* dXt = dX + (long long)t * M * Kr;
  const int kb = k0r + wm * S::WM + (lane >> 5) * 4;
  const int tok = m0 + wn * S::WN + (lane & 31);
#pragma unroll
  for (int i = 0; i < S::WI; ++i)
#pragma unroll
    for (int j = 0; j < S::WJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k = kb + i * 32 + q * 8, m = tok + j * 32;
        if (k < Kr && m < M) st8(dXt + (long long)m * Kr + k, pack4(acc[i][j], q));
      }
}

// ============================================================================
// Backward, weight gradient, computed as dW_t^T[c,k] = sum_m G_t[m,c] X_t[m,k].
// The contraction runs over tokens m, the strided index of both operands, so
// both are MNCONT: A = G_t ([m][c], staged through registers for the select),
// B = X_t ([m][k], copied directly).
// ============================================================================
template <int BM, int BN>
__global__ void __launch_bounds__(kGemmThreads, 1)
pcr_bwd_dw_kernel(const uint16_t* __restrict__ dZ, const uint16_t* __restrict__ Gs,
                  const uint16_t* __restrict__ X, const uint8_t* __restrict__ mask,
                  uint16_t* __restrict__ dW, int T, int M, int Kr, int H, int tiles_m, int tiles_n) {
  using S = TileShape<BM, BN>;
  constexpr int CPR = BM / 8;                   // 16-byte chunks per k-row of the A tile
  constexpr int NV = kBK * CPR / kGemmThreads;  // staged vectors per thread
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int per_rank = tiles_m * tiles_n;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int t = lin / per_rank;
  int tm, tn;
  tile_coords(lin - t * per_rank, tiles_m, tiles_n, tm, tn);
  const int c0 = tm * BM, k0r = tn * BN;  // channels (dW columns), rows of dW
  const long long MH = (long long)M * H, MK = (long long)M * Kr;
  const uint16_t* dZt = dZ + t * MH;
  const uint16_t* Xt = X + t * MK;
  const int nk = (M + kBK - 1) / kBK;
  const int kv_last = M - (nk - 1) * kBK;

  f32x16 acc[S::WI][S::WJ];
  zero_acc<BM, BN>(acc);

  // Staged A: this thread always owns channel chunk (tid % CPR) of the tile, so
  // its 8-channel select mask is loaded once.
  const int my_chunk = tid % CPR;
  const int ch = min(c0 + my_chunk * 8, H - 8);
  const u32x2 mk = *reinterpret_cast<const u32x2*>(mask + ch);
  const u32x4 sel = expand_mask8(mk[0], mk[1]);
  u32x4 vz[NV], vg[NV];
  auto load_a = [&](int c) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int m = min(c * kBK + (tid + i * kGemmThreads) / CPR, M - 1);
      const uint32_t off = (uint32_t)(m * H + ch);
      vz[i] = ld16(dZt + off);
      vg[i] = ld16(Gs + off);
    }
  };
  auto store_a = [&](int c, uint16_t* As) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int k = (tid + i * kGemmThreads) / CPR;
      st16(As + mn_off<BM>(k, my_chunk), c * kBK + k < M ? select8(vg[i], vz[i], sel) : z);
    }
  };
  const MnDma<BN> db(Xt, (uint32_t)(MK * 2), Kr, lane, wave);
  auto issue_b = [&](int c) { db.load(Kr, k0r, c * kBK, smem + (c & 1) * S::BUF + BM * kBK, wave); };

  load_a(0);
  issue_b(0);
  store_a(0, smem);
  for (int c = 0; c < nk; ++c) {
    uint16_t* As = smem + (c & 1) * S::BUF;
    uint16_t* Bs = As + BM * kBK;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const bool more = c + 1 < nk;
    if (more) {
      load_a(c + 1);
      issue_b(c + 1);
    }
    mma_chunk<BM, BN>([&](int ks, int i) { return frag_mncont<BM>(As, wm * S::WM + i * 32, ks, lane); },
                      [&](int ks, int j) { return frag_mncont<BN>(Bs, wn * S::WN + j * 32, ks, lane); }, acc);
    if (more) store_a(c + 1, smem + ((c + 1) & 1) * S::BUF);
  }

  uint16_t* dWt = dW + (long long)t * Kr * H;
  const int cb = c0 + wm * S::WM + (lane >> 5) * 4;
  const int kr = k0r + wn * S::WN + (lane & 31);
#pragma unroll
  for (int i = 0; i < S::WI; ++i)
#pragma unroll
    for (int j = 0; j < S::WJ; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = cb + i * 32 + q * 8, k = kr + j * 32;
        if (c < H && k < Kr) st8(dWt + (long long)k * H + c, pack4(acc[i][j], q));
      }
}

}  // namespace caat
