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
// the output's contiguous index); the epilogues restage it through LDS in row
// order and write whole lines with 16-byte stores.
#pragma once

#include <type_traits>

#include "gemm_core.hpp"
#include "reduce_kernels.hpp"

namespace caat {

// Opaque copy of a value: addresses derived from it are recomputed where they
// are used instead of being hoisted (and kept live) across the main loop.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

// A 64-bit value every lane holds the same copy of, made wave-uniform (scalar).
__device__ __forceinline__ unsigned long long uniform64(unsigned long long v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((unsigned long long)hi << 32) | lo;
}

// Orders this wave's LDS writes before its following LDS reads (and keeps the
// compiler from moving memory accesses across it).
__device__ __forceinline__ void lds_wave_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Which tiles a forward launch takes.  With a sync set that mixes synced and
// local channels inside 8-channel chunks (a random or strided S), the tiled
// kernel below writes those chunks twice (once at the rank's boundary, then
// the synced sums as partial lines); the register-queue kernel writes them
// once.  A launch can therefore be limited to the tiles whose 256-channel
// group of the mask holds such a chunk (kFwdMixed) or holds none
// (kFwdUniform), so that each kernel takes the groups it handles best.  The
// results are the same bits either way.
enum FwdMode { kFwdAll = 0, kFwdUniform = 1, kFwdMixed = 2 };

// Whether the 256-channel group of channel c0 has an 8-channel chunk with
// both synced and local channels (wave-uniform: all waves agree).
__device__ __forceinline__ bool mask_group_mixed(const uint8_t* __restrict__ mask, int c0, int H, int lane) {
  const int c = (c0 / kClassCols) * kClassCols + 8 * (lane & 31);
  bool mixed = false;
  if (lane < 32 && c < H) {  // H % 8 == 0: a chunk never straddles H
    const u32x2 w = *reinterpret_cast<const u32x2*>(mask + c);
    mixed = !(no_zero_byte(w[0]) && no_zero_byte(w[1])) && (w[0] | w[1]) != 0u;
  }
  return __any(mixed) != 0;
}

// Whether this workgroup's tile is outside the launch's share (all waves
// agree, so the workgroup leaves together, before any barrier).
__device__ __forceinline__ bool skip_tile(int mode, const uint8_t* __restrict__ mask, int c0, int H, int lane) {
  if (mode == kFwdAll || mask == nullptr) return false;
  return mask_group_mixed(mask, c0, H, lane) != (mode == kFwdMixed);
}

// ============================================================================
// Forward.  (mask == nullptr: no channel is synced, i.e. T independent
// products -- the column-parallel layer.)  One workgroup per (channel tile,
// token tile) walks the contraction
// of all T ranks in rank order.  Synced channels keep accumulating across the
// rank boundaries, so their fp32 accumulator ends as the sum over ranks
// (ascending t), formed once and written to every rank: bit-identical synced
// channels.  At the end of rank t < T-1 the tile is written to out[t] (its
// synced positions hold a partial sum there and are overwritten at the end)
// and the local accumulators restart from zero.  At the end the last rank's
// tile is written whole and the synced channels go to every other rank.
// A = W_t^T (channels x k, W is [k][c]: MNCONT); B = X_t (tokens x k: KCONT).
// All stores are staged through LDS so that they write whole lines: at a
// rank boundary through the LDS buffer of the chunk just consumed (the next
// chunk is landing in the other one), at the end through all of LDS.  They
// are non-temporal: the output is never re-read here, and streaming it past
// the caches keeps the operands' lines (and the end-of-tile partial-line
// writes) from contending with it (measured: 4-6% faster).
// ============================================================================
template <int BM, int BN, int NW>
__global__ void __launch_bounds__(NW * 64, 1)
rowpar_pcr_fwd_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                      const uint8_t* __restrict__ mask, uint16_t* __restrict__ out,
                      int T, int M, int Kr, int H, int tiles_m, int tiles_n, int mode) {
  using S = TileShape<BM, BN, NW>;
  using RS = RowStage<S::WM>;
  constexpr int REG = S::BUF / NW;             // boundary staging per wave (elements)
  constexpr int PASSES = (S::WM * S::WN + REG - 1) / REG;  // boundary passes over the wave's sub-tile
  constexpr int JPP = S::WJ / PASSES;                      // 32-token blocks per pass
  static_assert(PASSES * REG >= S::WM * S::WN && JPP * PASSES == S::WJ && JPP * 32 * S::WM <= REG, "staging split");
  static_assert(NW * S::WM * S::WN <= S::LDS_ELEMS, "final staging must fit");
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int c0 = tm * BM, m0 = tn * BN;  // channel tile, token tile
  if (skip_tile(mode, mask, c0, H, lane)) return;
  const int chw = c0 + wm * S::WM;       // this wave's first channel
  const int tkw = m0 + wn * S::WN;       // this wave's first token
  const int nk = (Kr + kBK - 1) / kBK;
  const int kv_last = Kr - (nk - 1) * kBK;  // valid k in a rank's last chunk
  const int nchunks = T * nk;
  const long long MK = (long long)M * Kr, KH = (long long)Kr * H, MH = (long long)M * H;

  // keepbits[i] has bit e set when accumulator register e of block i holds a
  // synced channel (channel chw + i*32 + (e/4)*8 + (lane/32)*4 + e%4).
  uint32_t keepbits[S::WI];
#pragma unroll
  for (int i = 0; i < S::WI; ++i) {
    uint32_t kb = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = chw + (lane >> 5) * 4 + i * 32 + q * 8;
      const uint32_t m4 = mask != nullptr && ch < H ? *reinterpret_cast<const uint32_t*>(mask + ch) : 0u;
#pragma unroll
      for (int r = 0; r < 4; ++r) kb |= ((m4 >> (8 * r)) & 0xffu) ? (1u << (4 * q + r)) : 0u;
    }
    keepbits[i] = kb;
  }

  // Mask of the 8-channel chunk this lane stores in every row-order drain
  // (bit b: channel chc + b synced).  A wholly synced chunk is skipped at the
  // rank boundaries: the end of the tile writes the synced sums over it.
  const int ccl = lane % RS::CPR;
  const int chc = chw + ccl * 8;
  uint32_t m8 = 0;
  if (mask != nullptr && chc < H) {
    const u32x2 mk = *reinterpret_cast<const u32x2*>(mask + chc);
#pragma unroll
    for (int b = 0; b < 8; ++b) m8 |= (((b < 4 ? mk[0] : mk[1]) >> (8 * (b & 3))) & 0xffu) ? (1u << b) : 0u;
  }

  f32x16 acc[S::WI][S::WJ];
  zero_acc<BM, BN, NW>(acc);

  auto issue = [&](int c) {
    const int t = c / nk;
    const int k0 = (c - t * nk) * kBK;
    uint16_t* buf = smem + (c & 1) * S::BUF;
    const MnDma<BM> da(W + t * KH, (uint32_t)(KH * 2), H, lane, wave);
    const KcDma db(X + t * MK, (uint32_t)(MK * 2), Kr, lane, wave);
    da.template load<NW>(H, c0, k0, buf, wave);
    db.load<BN, NW>(Kr, m0, k0, buf + BM * kBK, wave);
  };

  issue(0);
  for (int t = 0; t < T; ++t) {
    int c = t * nk;
    for (int kc = 0; kc < nk; ++kc, ++c) {
      uint16_t* As = smem + (c & 1) * S::BUF;
      uint16_t* Bs = As + BM * kBK;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (kc == nk - 1 && kv_last < kBK) {  // W's rows past Kr arrived as zeros
        zero_kcont_tail<BN, S::THREADS>(Bs, kv_last, tid);
        __syncthreads();
      }
      mma_chunk<BM, BN, NW>([&](int ks, int i) { return frag_mncont<BM>(As, wm * S::WM + i * 32, ks, lane); },
                        [&](int ks, int j) { return frag_kcont(Bs, wn * S::WN + j * 32, ks, lane); }, acc,
                        [&] {
                          if (c + 1 < nchunks) issue(c + 1);
                        });
    }
    if (t < T - 1) {
      // End of rank t < T-1: stage and write the tile to out[t], restart the
      // local channels.  The staging area is this wave's share of the buffer
      // the last chunk was read from.
      __syncthreads();
      uint16_t* st = smem + ((c - 1) & 1) * S::BUF + wave * REG;
      uint16_t* ot = out + t * MH;
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
#pragma unroll
        for (int jj = 0; jj < JPP; ++jj) {
          const int j = p * JPP + jj;
#pragma unroll
          for (int i = 0; i < S::WI; ++i) {
            RS::put(st, acc[i][j], i, jj * 32, lane);
            const uint32_t kb = (uint32_t)opaque((int)keepbits[i]);
#pragma unroll
            for (int e = 0; e < 16; ++e) {  // all ones where register e is a synced channel
              const uint32_t keep = (uint32_t)((int)(kb << (31 - e)) >> 31);
              acc[i][j][e] = __uint_as_float(__float_as_uint(acc[i][j][e]) & keep);
            }
            __builtin_amdgcn_sched_barrier(0);  // one block's registers at a time
          }
        }
        lds_wave_sync();
        const int tok0 = tkw + p * JPP * 32;
        RS::drain(st, JPP * 32, lane, [&](int r, int cc, u32x4 v) {
          const int tok = tok0 + r, ch = chw + cc * 8;
          if (tok < M && ch < H && m8 != 0xffu) st16_nt(ot + (long long)tok * H + ch, v);
        });
        lds_wave_sync();
      }
    }
  }

  // End of the tile: the accumulators now hold the synced channels' sums over
  // all ranks and the last rank's local channels, i.e. the last rank's output,
  // which is written whole; the synced sums then go to the synced positions
  // of every other rank, whose local positions were written at its boundary.
  __syncthreads();
  uint16_t* st = smem + wave * (S::WM * S::WN);
#pragma unroll
  for (int i = 0; i < S::WI; ++i)
#pragma unroll
    for (int j = 0; j < S::WJ; ++j) {
      RS::put(st, acc[i][j], i, j * 32, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  lds_wave_sync();
  // The earlier boundaries' stores cover lines written below: let them
  // complete first.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  {
    uint16_t* ol = out + (T - 1) * MH;
    RS::drain(st, S::WN, lane, [&](int r, int cc, u32x4 v) {
      const int tok = tkw + r, ch = chw + cc * 8;
      if (tok < M && ch < H) st16_nt(ol + (long long)tok * H + ch, v);
    });
  }
  if (T == 1 || mask == nullptr) return;  // nothing synced to hand to other ranks
  const int rows = min(S::WN, M - tkw);
  // When every chunk of the wave is all-synced or all-local, synced chunks
  // are written whole; otherwise each lane takes one channel and writes it
  // where synced (every synced channel, those of wholly synced chunks too).
  if (!__any(m8 != 0u && m8 != 0xffu)) {
    // Rank by rank: the output slices are M*H*2 bytes apart (128 MiB at the
    // Llama2-7B shape), so the T-1 copies of one row piece would fall on
    // the same HBM channels back to back; one rank's rows at a time spread
    // the stores over them (the LDS is read T-1 times).
    for (int u = 0; u < T - 1; ++u)
      RS::drain(st, S::WN, lane, [&](int r, int cc, u32x4 v) {
        if (m8 == 0xffu && r < rows) st16_nt(out + u * MH + (long long)(tkw + r) * H + chw + cc * 8, v);
      });
    return;
  }
#pragma unroll
  for (int h = 0; h < S::WM / 64; ++h) {
    const int cw = h * 64 + lane;  // channel within the sub-tile
    const int ch = chw + cw;
    if (ch < H && mask[ch] != 0) {
      const uint16_t* sp = st + (cw & 7);
      for (int u = 0; u < T - 1; ++u) {  // rank by rank, as above
        uint16_t* o = out + u * MH + (long long)tkw * H + ch;
        for (int r = 0; r < rows; ++r) {
          __builtin_nontemporal_store(sp[RS::off(r, cw >> 3)], o);
          o += H;
        }
      }
    }
  }
}

// ============================================================================
// Forward with the earlier ranks' tiles held in registers (2 <= T <= TB, the
// small tiles only).  The contraction is walked as in the kernel above (the
// same MFMAs in the same order), but at the end of rank t < T-1 each wave
// packs its accumulators to bf16 into a register queue and restarts the
// local channels: no LDS, barrier or store at a rank boundary.  At the end of
// the tile every rank's output is assembled in registers -- synced channels
// the sum, local channels that rank's own value -- and written once, whole
// lines through LDS.  Same bits as the kernel above; each output line is
// written once whatever S is (no second, partial-line write of the synced
// channels), and small contractions lose the per-rank drains.  The queue
// shifts by one slot per rank (static register indices), so the rank loop
// needs no unrolling.  It costs (T-1) x 16 registers per 32x32 block: with
// a 128x64 tile, T <= 4 keeps three workgroups per CU, T <= 8 two.
// ============================================================================
// (With TB = 8 the compiler is held to two workgroups per CU: a few rarely
// touched values then live in scratch, and the second workgroup hides the
// first one's latency -- T = 8, M = 8192, H = 768, Kr = 96: 67 -> 47 us, the
// same bits.  MINB = 3 holds it to three, with more values in scratch: that
// pays only where three per CU take every tile in one round and two would
// not, 513 to 768 tiles -- M = 8192, H = 768, Kr = 256 / 384 / 768: 75 / 91
// / 147 -> 63 / 75 / 113 us; with thousands of tiles it loses 5-8%.)
template <int BM, int BN, int NW, int TB, int MINB = (TB > 4 ? 2 : 1)>
__global__ void __launch_bounds__(NW * 64, MINB)
rowpar_pcr_fwd_rb_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                         const uint8_t* __restrict__ mask, uint16_t* __restrict__ out, int T, int M, int Kr, int H,
                         int tiles_m, int tiles_n, int mode) {
  using S = TileShape<BM, BN, NW>;
  using RS = RowStage<S::WM>;
  static_assert(TB >= 2 && TB <= 8, "ranks held in registers");
  static_assert(NW * S::WM * S::WN <= S::LDS_ELEMS, "final staging must fit");
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  int tm, tn;
  tile_coords(xcd_remap(blockIdx.x, gridDim.x), tiles_m, tiles_n, tm, tn);
  const int c0 = tm * BM, m0 = tn * BN;  // channel tile, token tile
  if (skip_tile(mode, mask, c0, H, lane)) return;
  const int chw = c0 + wm * S::WM;       // this wave's first channel
  const int tkw = m0 + wn * S::WN;       // this wave's first token
  const int nk = (Kr + kBK - 1) / kBK;
  const int kv_last = Kr - (nk - 1) * kBK;
  const int nchunks = T * nk;
  const long long MK = (long long)M * Kr, KH = (long long)Kr * H, MH = (long long)M * H;

  // keepbits[i] bit e: accumulator register e of block i holds a synced
  // channel (the same layout as in the kernel above).
  uint32_t keepbits[S::WI];
#pragma unroll
  for (int i = 0; i < S::WI; ++i) {
    uint32_t kb = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ch = chw + (lane >> 5) * 4 + i * 32 + q * 8;
      const uint32_t m4 = ch < H ? *reinterpret_cast<const uint32_t*>(mask + ch) : 0u;
#pragma unroll
      for (int r = 0; r < 4; ++r) kb |= ((m4 >> (8 * r)) & 0xffu) ? (1u << (4 * q + r)) : 0u;
    }
    keepbits[i] = kb;
  }

  f32x16 acc[S::WI][S::WJ];
  zero_acc<BM, BN, NW>(acc);
  // Queue of the finished ranks' tiles (bf16 pairs): slot 0 is the latest
  // rank; after the loop slot k holds rank T-2-k.
  uint32_t pk[TB - 1][S::WI][S::WJ][8] = {};

  auto issue = [&](int c) {
    const int t = c / nk;
    const int k0 = (c - t * nk) * kBK;
    uint16_t* buf = smem + (c & 1) * S::BUF;
    const MnDma<BM> da(W + t * KH, (uint32_t)(KH * 2), H, lane, wave);
    const KcDma db(X + t * MK, (uint32_t)(MK * 2), Kr, lane, wave);
    da.template load<NW>(H, c0, k0, buf, wave);
    db.load<BN, NW>(Kr, m0, k0, buf + BM * kBK, wave);
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
        zero_kcont_tail<BN, S::THREADS>(Bs, kv_last, tid);
        __syncthreads();
      }
      mma_chunk<BM, BN, NW>([&](int ks, int i) { return frag_mncont<BM>(As, wm * S::WM + i * 32, ks, lane); },
                            [&](int ks, int j) { return frag_kcont(Bs, wn * S::WN + j * 32, ks, lane); }, acc,
                            [&] {
                              if (c + 1 < nchunks) issue(c + 1);
                            });
    }
    if (t < T - 1) {  // rank t's tile into the queue; the local channels restart
#pragma unroll
      for (int k = TB - 2; k >= 1; --k)
#pragma unroll
        for (int i = 0; i < S::WI; ++i)
#pragma unroll
          for (int j = 0; j < S::WJ; ++j)
#pragma unroll
            for (int w = 0; w < 8; ++w) pk[k][i][j][w] = pk[k - 1][i][j][w];
#pragma unroll
      for (int i = 0; i < S::WI; ++i)
#pragma unroll
        for (int j = 0; j < S::WJ; ++j) {
#pragma unroll
          for (int w = 0; w < 8; ++w) pk[0][i][j][w] = pack_bf16x2(acc[i][j][2 * w], acc[i][j][2 * w + 1]);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const uint32_t keep = (uint32_t)((int)(keepbits[i] << (31 - e)) >> 31);
            acc[i][j][e] = __uint_as_float(__float_as_uint(acc[i][j][e]) & keep);
          }
        }
    }
  }

  // The accumulators hold the synced sums and the last rank's local values.
  __syncthreads();  // every wave is done with the operand buffers
  uint16_t* st = smem + wave * (S::WM * S::WN);
  // Ranks T-1, T-2, ..., 0: the last straight from the accumulators, each
  // earlier one the sums on synced channels and queue slot 0 elsewhere; the
  // queue then shifts down.
  for (int u = T - 1; u >= 0; --u) {
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int j = 0; j < S::WJ; ++j) {
        uint32_t v[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
          const uint32_t sw = pack_bf16x2(acc[i][j][2 * w], acc[i][j][2 * w + 1]);
          const uint32_t km = (((keepbits[i] >> (2 * w)) & 1u) ? 0xffffu : 0u) |
                              (((keepbits[i] >> (2 * w + 1)) & 1u) ? 0xffff0000u : 0u);
          v[w] = u == T - 1 ? sw : (sw & km) | (pk[0][i][j][w] & ~km);
        }
        RS::put_packed(st, v, i, j * 32, lane);
      }
    if (u < T - 1) {
#pragma unroll
      for (int k = 0; k + 1 < TB - 1; ++k)
#pragma unroll
        for (int i = 0; i < S::WI; ++i)
#pragma unroll
          for (int j = 0; j < S::WJ; ++j)
#pragma unroll
            for (int w = 0; w < 8; ++w) pk[k][i][j][w] = pk[k + 1][i][j][w];
    }
    lds_wave_sync();
    uint16_t* ou = out + u * MH;
    RS::drain(st, S::WN, lane, [&](int r, int cc, u32x4 v) {
      const int tok = tkw + r, ch = chw + cc * 8;
      if (tok < M && ch < H) st16_nt(ou + (long long)tok * H + ch, v);
    });
    lds_wave_sync();  // the drain's reads are done before the next rank's puts
  }
}

// ============================================================================
// Backward.  G_t (the reduced incoming gradient: the sum over ranks on synced
// channels, rank t's own gradient elsewhere -- the same partial channel-reduce
// applied to dZ) is materialised beforehand for every rank, so both products
// read plain operands copied straight into LDS.
//
// Input gradient, computed as dX_t^T[k,m] = sum_c W_t[k,c] G_t[m,c]:
// A = W_t (rows k, contraction over channels c contiguous: KCONT);
// B = G_t (rows m: KCONT).
// ============================================================================
template <int BM, int BN, int NW>
__global__ void __launch_bounds__(NW * 64, 1)
pcr_bwd_dx_kernel(const uint16_t* __restrict__ G, const uint16_t* __restrict__ W, uint16_t* __restrict__ dX,
                  int T, int M, int Kr, int H, int tiles_m, int tiles_n, const uint16_t* __restrict__ dZ,
                  const unsigned long long* __restrict__ tbits) {
  using S = TileShape<BM, BN, NW>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int per_rank = tiles_m * tiles_n;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int t = lin / per_rank;
  int tm, tn;
  tile_coords(lin - t * per_rank, tiles_m, tiles_n, tm, tn);
  const int k0r = tm * BM, m0 = tn * BN;  // rows of W_t (dX columns), tokens
  const long long MH = (long long)M * H, KH = (long long)Kr * H;
  const int nk = (H + kBK - 1) / kBK;
  const int kv_last = H - (nk - 1) * kBK;

  f32x16 acc[S::WI][S::WJ];
  zero_acc<BM, BN, NW>(acc);

  const KcDma da(W + t * KH, (uint32_t)(KH * 2), H, lane, wave);
  KcDma db(G + t * MH, (uint32_t)(MH * 2), H, lane, wave);
  // With tile classes, chunk c's columns of G_t come from dZ_t (a wholly
  // local tile of channels), from rank 0's slot (wholly synced: the one sum)
  // or from G_t itself (mixed); the three buffers share one layout.
  unsigned long long sbits = 0, lbits = 0;
  if (tbits != nullptr) {
    sbits = uniform64(tbits[0]);
    lbits = uniform64(tbits[1]);
  }
  auto issue = [&](int c) {
    uint16_t* buf = smem + (c & 1) * S::BUF;
    if (tbits != nullptr) {
      const int tile = (c * kBK) / kClassCols;
      const uint16_t* src = ((lbits >> tile) & 1ull) ? dZ + t * MH : ((sbits >> tile) & 1ull) ? G : G + t * MH;
      db.rsrc = make_rsrc((const void*)uniform64((unsigned long long)(uintptr_t)src), (uint32_t)(MH * 2));
    }
    da.load<BM, NW>(H, k0r, c * kBK, buf, wave);
    db.load<BN, NW>(H, m0, c * kBK, buf + BM * kBK, wave);
  };

  // A wave whose rows of dX_t^T all lie past Kr (the last column tile when
  // Kr is not a multiple of BM) only issues its share of the copies.  Waves
  // with the same wm sit on different SIMDs, so the idle ones free half of
  // every SIMD's matrix-core time in such a tile.
  // (The two kinds of wave run separate copies of the loop, with the same
  // barriers, so that neither carries the other's registers.)
  auto loop = [&](auto compute) {
    issue(0);
    for (int c = 0; c < nk; ++c) {
      uint16_t* As = smem + (c & 1) * S::BUF;
      uint16_t* Bs = As + BM * kBK;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (c == nk - 1 && kv_last < kBK) {  // channels past H: the next row's values
        zero_kcont_tail<BM, S::THREADS>(As, kv_last, tid);
        zero_kcont_tail<BN, S::THREADS>(Bs, kv_last, tid);
        __syncthreads();
      }
      if constexpr (decltype(compute)::value)
        mma_chunk<BM, BN, NW>([&](int ks, int i) { return frag_kcont(As, wm * S::WM + i * 32, ks, lane); },
                          [&](int ks, int j) { return frag_kcont(Bs, wn * S::WN + j * 32, ks, lane); }, acc,
                          [&] {
                            if (c + 1 < nk) issue(c + 1);
                          });
      else if (c + 1 < nk)
        issue(c + 1);
    }
  };
  if (k0r + wm * S::WM < Kr)
    loop(std::true_type{});
  else
    loop(std::false_type{});

  // Stage the transposed sub-tile through LDS and write whole rows of dX_t.
  using RS = RowStage<S::WM>;
  __syncthreads();
  uint16_t* st = smem + wave * (S::WM * S::WN);
#pragma unroll
  for (int i = 0; i < S::WI; ++i)
#pragma unroll
    for (int j = 0; j < S::WJ; ++j) {
      RS::put(st, acc[i][j], i, j * 32, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  lds_wave_sync();
  uint16_t* dXt = dX + (long long)t * M * Kr;
  const int kw = k0r + wm * S::WM, mw = m0 + wn * S::WN;
  RS::drain(st, S::WN, lane, [&](int r, int cc, u32x4 v) {
    const int m = mw + r, k = kw + cc * 8;
    if (m < M && k < Kr) st16(dXt + (long long)m * Kr + k, v);
  });
}

// ============================================================================
// Weight gradient, computed as dW_t^T[c,k] = sum_m G_t[m,c] X_t[m,k].  The
// contraction runs over tokens m, the strided index of both operands, so both
// are MNCONT: A = G_t ([m][c]), B = X_t ([m][k]).  Token rows past M read as
// zero (outside the rank's buffer).
// ============================================================================
//
// SPLIT: when dW_t has too few tiles to fill the chip, the token range is cut
// into `splits` pieces of `kcs` chunks; workgroup (t, piece, tile) leaves its
// fp32 sum over its piece in part[piece][t][k][c], and dw_split_sum_kernel
// adds the pieces in order and rounds once.
template <int BM, int BN, int NW, bool SPLIT = false>
__global__ void __launch_bounds__(NW * 64, 1)
pcr_bwd_dw_kernel(const uint16_t* __restrict__ G, const uint16_t* __restrict__ X, uint16_t* __restrict__ dW,
                  int T, int M, int Kr, int H, int tiles_m, int tiles_n, float* __restrict__ part, int splits,
                  int kcs, const uint16_t* __restrict__ dZ, const unsigned long long* __restrict__ tbits) {
  using S = TileShape<BM, BN, NW>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // wn = wave / 2: the two waves of each SIMD (wave and wave + 4 with eight
  // waves) take different row ranges of dW_t, so when the last row tile
  // leaves the upper waves idle (below) every SIMD keeps one busy wave.
  const int wm = wave % S::WGM, wn = wave / S::WGM;
  const int per_rank = tiles_m * tiles_n;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int t = lin / (splits * per_rank);
  const int rest = lin - t * splits * per_rank;
  const int piece = rest / per_rank;
  int tm, tn;
  tile_coords(rest - piece * per_rank, tiles_m, tiles_n, tm, tn);
  const int c0 = tm * BM, k0r = tn * BN;  // channels (dW columns), rows of dW
  const long long MH = (long long)M * H, MK = (long long)M * Kr;
  const int nkm = (M + kBK - 1) / kBK;
  const int cb = piece * kcs;                       // this piece's chunks: cb .. ce-1
  const int ce = cb + kcs < nkm ? cb + kcs : nkm;

  f32x16 acc[S::WI][S::WJ];
  zero_acc<BM, BN, NW>(acc);

  // With tile classes, this tile's channels of G_t come from dZ_t (wholly
  // local), from rank 0's slot (wholly synced) or from G_t (mixed).  BM <= 256
  // and c0 is a multiple of BM, so the tile lies in one class tile.
  const uint16_t* gsrc = G + t * MH;
  if (tbits != nullptr) {
    const int tile = c0 / kClassCols;
    if ((uniform64(tbits[1]) >> tile) & 1ull)
      gsrc = dZ + t * MH;
    else if ((uniform64(tbits[0]) >> tile) & 1ull)
      gsrc = G;
    gsrc = (const uint16_t*)uniform64((unsigned long long)(uintptr_t)gsrc);
  }
  const MnDma<BM> da(gsrc, (uint32_t)(MH * 2), H, lane, wave);
  const MnDma<BN> db(X + t * MK, (uint32_t)(MK * 2), Kr, lane, wave);
  auto issue = [&](int c) {
    uint16_t* buf = smem + (c & 1) * S::BUF;
    da.template load<NW>(H, c0, c * kBK, buf, wave);
    db.template load<NW>(Kr, k0r, c * kBK, buf + BM * kBK, wave);
  };

  // A wave whose rows of dW_t all lie past Kr (the last row tile when Kr is
  // not a multiple of BN) only issues its share of the copies.
  auto loop = [&](auto compute) {
    issue(cb);
    for (int c = cb; c < ce; ++c) {
      uint16_t* As = smem + (c & 1) * S::BUF;
      uint16_t* Bs = As + BM * kBK;
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if constexpr (decltype(compute)::value)
        mma_chunk<BM, BN, NW>([&](int ks, int i) { return frag_mncont<BM>(As, wm * S::WM + i * 32, ks, lane); },
                          [&](int ks, int j) { return frag_mncont<BN>(Bs, wn * S::WN + j * 32, ks, lane); }, acc,
                          [&] {
                            if (c + 1 < ce) issue(c + 1);
                          });
      else if (c + 1 < ce)
        issue(c + 1);
    }
  };
  if (k0r + wn * S::WN < Kr)
    loop(std::true_type{});
  else
    loop(std::false_type{});

  const int cw = c0 + wm * S::WM, kw = k0r + wn * S::WN;
  if constexpr (SPLIT) {
    // fp32 piece sums straight from the accumulators: register group q of
    // block (i, j) holds channels cw + 32i + 8q + 4(lane/32) .. +3 of dW row
    // kw + 32j + lane%32 (16 contiguous bytes).
    float* pt = part + ((long long)piece * T + t) * Kr * H;
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int j = 0; j < S::WJ; ++j) {
        const int k = kw + j * 32 + (lane & 31);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = cw + i * 32 + q * 8 + (lane >> 5) * 4;
          if (k < Kr && c < H) {
            f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            *reinterpret_cast<f32x4*>(pt + (long long)k * H + c) = v;
          }
        }
      }
    return;
  }

  // Stage the transposed sub-tile through LDS and write whole rows of dW_t.
  using RS = RowStage<S::WM>;
  __syncthreads();
  uint16_t* st = smem + wave * (S::WM * S::WN);
#pragma unroll
  for (int i = 0; i < S::WI; ++i)
#pragma unroll
    for (int j = 0; j < S::WJ; ++j) {
      RS::put(st, acc[i][j], i, j * 32, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
  lds_wave_sync();
  uint16_t* dWt = dW + (long long)t * Kr * H;
  RS::drain(st, S::WN, lane, [&](int r, int cc, u32x4 v) {
    const int k = kw + r, c = cw + cc * 8;
    if (k < Kr && c < H) st16(dWt + (long long)k * H + c, v);
  });
}

// dW = the sum of the pieces' fp32 partials in piece order, rounded once to
// bf16: four consecutive elements per thread (n4 = T*Kr*H/4 groups).
__global__ void dw_split_sum_kernel(const float* __restrict__ part, uint16_t* __restrict__ dW, int splits,
                                    long long n4) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const f32x4* p = reinterpret_cast<const f32x4*>(part) + i;
  f32x4 v = p[0];
  for (int s = 1; s < splits; ++s) v += p[(long long)s * n4];
  u32x2 o;
  o[0] = pack_bf16x2(v[0], v[1]);
  o[1] = pack_bf16x2(v[2], v[3]);
  reinterpret_cast<u32x2*>(dW)[i] = o;
}

}  // namespace caat
