// bf16 MFMA GEMM building blocks for gfx950 (CDNA4).
//
// A workgroup of 256 threads (4 wave64s in a 2x2 grid) owns a BM x BN output
// tile and walks the contraction in 64-wide chunks.  Each chunk of both
// operands is staged through LDS as [row][64 k] bf16 rows (see lds_off), double
// buffered, with the next chunk's global loads in flight while the current one
// feeds v_mfma_f32_32x32x16_bf16 (fp32 accumulation).
//
// Operands are described by where their contraction index is contiguous:
//   * KCONT:  memory [row][k], k contiguous  -> 16-byte vectors copied as is;
//   * MNCONT: memory [k][row], row contiguous -> 8x8 blocks loaded as 8 rows of
//             16 bytes and transposed in registers before the LDS write.
#pragma once

#include "common.hpp"

namespace caat {

constexpr int kGemmThreads = 256;
constexpr int kBK = 64;

template <int BM, int BN>
struct TileShape {
  static constexpr int WM = BM / 2, WN = BN / 2;    // per-wave sub-tile (2x2 waves)
  static constexpr int WI = WM / 32, WJ = WN / 32;  // 32x32 MFMA blocks per wave
  static constexpr int LDS_ELEMS = 2 * (BM + BN) * kBK;  // double buffer, bf16 elements
  static_assert(BM % 64 == 0 && BN % 64 == 0, "tile must be a multiple of 64");
};

// ---- KCONT loader: R rows x 64 k, one 16-byte vector per (row, k-chunk) -------
template <int R>
struct KContLoader {
  static constexpr int NV = (R * 8 + kGemmThreads - 1) / kGemmThreads;
  u32x4 v[NV];

  // src(row, k) returns the 16-byte vector of 8 k-values at (row, k..k+7) or
  // zero; the caller clamps rows and zero-fills k beyond the contraction.
  template <class Src>
  __device__ __forceinline__ void load(Src&& src, int tid) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int q = tid + i * kGemmThreads;
      if (R * 8 % kGemmThreads == 0 || q < R * 8) v[i] = src(q >> 3, (q & 7) * 8);
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int q = tid + i * kGemmThreads;
      if (R * 8 % kGemmThreads == 0 || q < R * 8) st16(lds + lds_off(q >> 3, q & 7), v[i]);
    }
  }
};

// ---- MNCONT loader: 64 k x R rows held as [k][row]; 8x8 blocks per thread -----
template <int R>
struct MNContLoader {
  static constexpr int NBLK = (kBK / 8) * (R / 8);
  static constexpr int NB = (NBLK + kGemmThreads - 1) / kGemmThreads;
  u32x4 v[NB][8];

  // src(kk, row) returns 8 consecutive rows' values at contraction index kk
  // (16 bytes), or zero beyond the contraction.
  template <class Src>
  __device__ __forceinline__ void load(Src&& src, int tid) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int q = tid + b * kGemmThreads;
      if (NBLK % kGemmThreads == 0 || q < NBLK) {
        const int rb = q % (R / 8), kb = q / (R / 8);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[b][i] = src(kb * 8 + i, rb * 8);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* lds, int tid) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int q = tid + b * kGemmThreads;
      if (NBLK % kGemmThreads == 0 || q < NBLK) {
        const int rb = q % (R / 8), kb = q / (R / 8);
        u32x4 o[8];
        transpose8x8(v[b], o);
#pragma unroll
        for (int j = 0; j < 8; ++j) st16(lds + lds_off(rb * 8 + j, kb), o[j]);
      }
    }
  }
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// One 64-wide chunk of MFMAs for this wave's WI x WJ blocks.
template <int BM, int BN>
__device__ __forceinline__ void mma_chunk(const uint16_t* As, const uint16_t* Bs, int wm, int wn, int lane,
                                          f32x16 (&acc)[TileShape<BM, BN>::WI][TileShape<BM, BN>::WJ]) {
  using S = TileShape<BM, BN>;
  const int r = lane & 31;
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    const int kc = ks * 2 + (lane >> 5);
    u32x4 a[S::WI], b[S::WJ];
#pragma unroll
    for (int i = 0; i < S::WI; ++i) a[i] = ld16(As + lds_off(wm * S::WM + i * 32 + r, kc));
#pragma unroll
    for (int j = 0; j < S::WJ; ++j) b[j] = ld16(Bs + lds_off(wn * S::WN + j * 32 + r, kc));
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int j = 0; j < S::WJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[i]), as_bf16x8(b[j]), acc[i][j], 0, 0, 0);
  }
}

// Row (within the 32x32 block) of accumulator register e of lane `lane`; the
// column is lane % 32.
__device__ __forceinline__ int acc_row(int e, int lane) { return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3); }

// Grouped raster of a tiles_m x tiles_n grid: GROUP m-tiles are walked
// column by column, so consecutive tiles share B columns and nearby A rows.
__device__ __forceinline__ void tile_coords(int tile, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int g = tile / per_group;
  const int first = g * GROUP;
  const int gsz = min(tiles_m - first, GROUP);
  const int in = tile - g * per_group;
  tm = first + in % gsz;
  tn = in / gsz;
}

// The double-buffered main loop.  load(c) issues chunk c's global loads into
// registers, store(a_lds, b_lds) writes them to LDS; after chunk c's MFMAs,
// after_chunk(c) runs (the forward uses it at rank boundaries).
template <int BM, int BN, class Load, class Store, class After>
__device__ __forceinline__ void gemm_mainloop(uint16_t* smem, int nchunks, Load&& load, Store&& store,
                                              After&& after_chunk,
                                              f32x16 (&acc)[TileShape<BM, BN>::WI][TileShape<BM, BN>::WJ]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int BUF = (BM + BN) * kBK;
  if (nchunks <= 0) return;
  load(0);
  store(smem, smem + BM * kBK);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    uint16_t* cur = smem + (c & 1) * BUF;
    uint16_t* nxt = smem + ((c + 1) & 1) * BUF;
    const bool more = c + 1 < nchunks;
    if (more) load(c + 1);
    mma_chunk<BM, BN>(cur, cur + BM * kBK, wm, wn, lane, acc);
    if (more) store(nxt, nxt + BM * kBK);
    after_chunk(c);
    __syncthreads();
  }
}


// Forward variant of the main loop: the contraction is T ranks of nk chunks.
// Between ranks, at_rank_end(t) runs once (outside the inner chunk loop, so
// the inner loop's accumulators stay in MFMA accumulation registers).
template <int BM, int BN, class Load, class Store, class RankEnd>
__device__ __forceinline__ void gemm_mainloop_ranks(uint16_t* smem, int T, int nk, Load&& load, Store&& store,
                                                    RankEnd&& at_rank_end,
                                                    f32x16 (&acc)[TileShape<BM, BN>::WI][TileShape<BM, BN>::WJ]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int BUF = (BM + BN) * kBK;
  const int nchunks = T * nk;
  if (nchunks <= 0) return;
  load(0);
  store(smem, smem + BM * kBK);
  __syncthreads();
  int c = 0;
  for (int t = 0; t < T; ++t) {
    for (int kc = 0; kc < nk; ++kc, ++c) {
      uint16_t* cur = smem + (c & 1) * BUF;
      uint16_t* nxt = smem + ((c + 1) & 1) * BUF;
      const bool more = c + 1 < nchunks;
      if (more) load(c + 1);
      mma_chunk<BM, BN>(cur, cur + BM * kBK, wm, wn, lane, acc);
      if (more) store(nxt, nxt + BM * kBK);
      __syncthreads();
    }
    if (t + 1 < T) at_rank_end(t);
  }
}

}  // namespace caat
