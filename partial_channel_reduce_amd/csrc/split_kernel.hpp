// Forward for token counts between decode and full tiles (the rank walk
// split across workgroups).
//
// The fused forward gives each (channel tile, token tile) to one workgroup,
// which walks all T ranks' contractions in turn.  With a few hundred tokens
// that leaves too few tiles to fill the chip, each with a long serial walk.
// Here every (rank t, channel block, token block) is a workgroup of its own
// (tiles of 128 x 64, 128 x 128 or 256 x 256; with few tiles and a long
// contraction, one workgroup per slice of it) and computes only Y_t's tile
// (the same copy and MFMA loop as the fused forward, over rank t's
// contraction):
//   * with no mask (the column-parallel layer: nothing synced) it writes the
//     tile to out[t] in bf16;
//   * otherwise it writes the fp32 tile to Y[t] in the workspace, and a
//     second kernel, pcr_reduce_f32_bf16_kernel, forms the partial
//     channel-reduce of Y into out: on synced channels the fp32 sum over the
//     ranks in ascending order, starting from rank 0's value, rounded once
//     (the same value on every rank); elsewhere the rank's own value.  With
//     whole contractions (ks == 1) and H a multiple of 64, a 64-channel group
//     with no synced channel needs no sum: it goes straight to out[t] in bf16
//     (the same rounding of the same value), and the second pass skips it,
//     so a contiguous sync set moves half the fp32 bytes (a scattered one
//     leaves practically no such group).
// Per-rank products are fp32 MFMA sums over that rank's contraction (CAAT-Net
// paper, Introduction: only the channels of the sync set are reduced over the
// tensor-parallel ranks).  The kernel boundary orders the two passes, so no
// cross-workgroup handoff is needed: the fp32 tiles go out with plain stores,
// and the four 16-byte stores that cover each 128-byte row piece merge into
// whole lines in L2.
#pragma once

#include "gemm_core.hpp"

namespace caat {

// Tiles: 128 channels x 64 or 128 tokens, four waves.
constexpr int kSplitBM = 128;
constexpr int kSplitNW = 4;

// With ks > 1 (fp32 products only) each rank's contraction is cut into ks
// slices of whole chunks, one workgroup each, and slice q of rank t goes to
// Y[q][t]; the second pass adds a rank's slices in slice order first.
template <int BM, int BN, int NW>
__global__ void __launch_bounds__(NW * 64, 1)
rowpar_pcr_split_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W, uint16_t* __restrict__ out,
                        float* __restrict__ Y, int T, int M, int Kr, int H, int tiles_m, int tiles_n, int ks,
                        const uint8_t* __restrict__ local_mask) {
  using S = TileShape<BM, BN, NW>;
  using RS = RowStage<S::WM>;
  static_assert(NW * S::WM * S::WN <= S::LDS_ELEMS, "final staging must fit");
  __shared__ __attribute__((aligned(16))) uint16_t smem[S::LDS_ELEMS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / S::WGN, wn = wave % S::WGN;
  const int per_rank = tiles_m * tiles_n;
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int tq = lin / per_rank;  // t * ks + q
  const int t = tq / ks, q = tq - t * ks;
  const int tile = lin - tq * per_rank;
  int tm, tn;
  tile_coords(tile, tiles_m, tiles_n, tm, tn);
  const int c0 = tm * BM, m0 = tn * BN;  // channel block, token block
  const int chw = c0 + wm * S::WM;       // this wave's first channel
  const int tkw = m0 + wn * S::WN;       // this wave's first token
  const int nk = (Kr + kBK - 1) / kBK;
  const int kv_last = Kr - (nk - 1) * kBK;
  const int kcs = (nk + ks - 1) / ks;              // chunks per slice
  const int cb = q * kcs, ce = min(nk, cb + kcs);  // this slice: chunks cb .. ce-1 (none past nk)
  const long long MK = (long long)M * Kr, KH = (long long)Kr * H, MH = (long long)M * H;

  f32x16 acc[S::WI][S::WJ];
  zero_acc<BM, BN, NW>(acc);
  const MnDma<BM> da(W + t * KH, (uint32_t)(KH * 2), H, lane, wave);
  const KcDma db(X + t * MK, (uint32_t)(MK * 2), Kr, lane, wave);
  auto issue = [&](int c) {
    uint16_t* buf = smem + (c & 1) * S::BUF;
    da.template load<NW>(H, c0, c * kBK, buf, wave);
    db.load<BN, NW>(Kr, m0, c * kBK, buf + BM * kBK, wave);
  };
  if (cb < ce) issue(cb);
  for (int c = cb; c < ce; ++c) {
    uint16_t* As = smem + (c & 1) * S::BUF;
    uint16_t* Bs = As + BM * kBK;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (c == nk - 1 && kv_last < kBK) {  // X's columns past Kr: the next row's values
      zero_kcont_tail<BN, S::THREADS>(Bs, kv_last, tid);
      __syncthreads();
    }
    mma_chunk<BM, BN, NW>([&](int ks, int i) { return frag_mncont<BM>(As, wm * S::WM + i * 32, ks, lane); },
                          [&](int ks, int j) { return frag_kcont(Bs, wn * S::WN + j * 32, ks, lane); }, acc,
                          [&] {
                            if (c + 1 < ce) issue(c + 1);
                          });
  }

  __syncthreads();  // every wave is done with the operand buffers
  if (Y == nullptr) {
    // bf16 straight to out[t], staged through this wave's part of LDS and
    // written as whole lines
    uint16_t* st = smem + wave * (S::WM * S::WN);
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int j = 0; j < S::WJ; ++j) RS::put(st, acc[i][j], i, j * 32, lane);
    lds_wave_sync();
    uint16_t* ou = out + t * MH;
    RS::drain(st, S::WN, lane, [&](int r, int cc, u32x4 w) {
      const int tok = tkw + r, ch = chw + cc * 8;
      if (tok < M && ch < H) st16_nt(ou + (long long)tok * H + ch, w);
    });
    return;
  }
  // fp32 to Y[q][t]: accumulator registers 4r..4r+3 of block (i, j) are 4
  // consecutive channels of one token, lanes l and l + 32 the two halves of
  // the 8-channel chunk chw + 32 i + 8 r.  With local_mask (whole
  // contractions, H a multiple of 64) a 64-channel group with no synced
  // channel goes to out[t] in bf16 instead, staged through this wave's part
  // of LDS and written as whole lines.  The group flags depend on the wave's
  // channels only, so the choice is uniform across its lanes.
  constexpr int NG = S::WM / 64;  // 64-channel groups per wave: 1 or 2
  static_assert(NG == 1 || NG == 2, "wave channel extent");
  float* yt = Y + ((long long)q * T + t) * MH;
  // Lane l reads mask word l % 8 (8 channels) of group (l / 8) % NG; a
  // group is direct when no lane of it saw a synced channel.
  bool loc64[NG];
  bool stage = false;
  {
    const int gl = (lane >> 3) & (NG - 1), cl = chw + 64 * gl + 8 * (lane & 7);
    bool syn = true;
    if (local_mask != nullptr && chw + 64 * gl < H) {
      syn = false;
      if (cl < H) {
        const u32x2 m8 = *reinterpret_cast<const u32x2*>(local_mask + cl);
        syn = (m8[0] | m8[1]) != 0u;
      }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      loc64[g] = !__any(syn && gl == g);
      stage |= loc64[g];
    }
  }
  if (stage) {
    uint16_t* st = smem + wave * (S::WM * S::WN);
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int j = 0; j < S::WJ; ++j) RS::put(st, acc[i][j], i, j * 32, lane);
    lds_wave_sync();
    uint16_t* ou = out + t * MH;
    RS::drain(st, S::WN, lane, [&](int r, int cc, u32x4 w) {
      const int tok = tkw + r, ch = chw + cc * 8;
      const bool direct = NG == 1 || cc * 8 < 64 ? loc64[0] : loc64[NG - 1];
      if (direct && tok < M && ch < H) st16_nt(ou + (long long)tok * H + ch, w);
    });
  }
#pragma unroll
  for (int i = 0; i < S::WI; ++i)
#pragma unroll
    for (int j = 0; j < S::WJ; ++j) {
      const int tok = tkw + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ch = chw + i * 32 + r * 8 + (lane >> 5) * 4;
        const bool direct = loc64[(i * 32 + r * 8) / 64];
        const f32x4 v = {acc[i][j][4 * r], acc[i][j][4 * r + 1], acc[i][j][4 * r + 2], acc[i][j][4 * r + 3]};
        if (!direct && tok < M && ch < H) *reinterpret_cast<f32x4*>(yt + (long long)tok * H + ch) = v;
      }
    }
}

}  // namespace caat

