// C ABI of the partial channel-reduce library: host-side validation and kernel
// dispatch.  Declarations and the contract of every call are in caat_pcr.h.
#include "caat_pcr.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "decode_kernel.hpp"
#include "gemm_kernels.hpp"
#include "norm_kernels.hpp"
#include "reduce_kernels.hpp"
#include "split_kernel.hpp"

namespace {

using namespace caat;

constexpr int kMaxT = 64;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int check_dims(int T, int M, int Kr, int H) {
  if (T < 1 || T > kMaxT || M < 0 || Kr < 8 || H < 8) return CAAT_ERR_DIM;
  if (Kr % 8 != 0 || H % 8 != 0) return CAAT_ERR_DIM;
  // element counts of the largest tensor must fit the kernels' 64-bit offsets
  // and the grid sizes (<= 2^31 workgroups)
  if ((long long)T * M * (long long)(H > Kr ? H : Kr) > (1LL << 40)) return CAAT_ERR_DIM;
  // one rank's bf16 slices are addressed with 32-bit signed byte offsets
  const long long lim = 1LL << 30;
  if ((long long)M * Kr >= lim || (long long)Kr * H >= lim || (long long)M * H >= lim) return CAAT_ERR_DIM;
  return CAAT_OK;
}

int launched() { return hipGetLastError() == hipSuccess ? CAAT_OK : CAAT_ERR_LAUNCH; }

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Waves per workgroup of the 256x256-tile GEMMs: eight (two per SIMD, each
// with a 128x64 sub-tile) hide LDS and barrier waits behind the other wave's
// MFMAs; the 128x128 tiles of small problems keep four.
constexpr int kBigTileWaves = 8;

// Compute units of the MI355X: one round of one-per-CU workgroups.
constexpr int kCUs = 256;

// The fused forward's 256 x 256 tiles: from this many of them (see
// fwd_launch).
constexpr int kFwdBigTiles = 160;

// 256 x 256 tiles (eight waves) when there are at least as many as CUs,
// else 128 x 128 (four waves).  (At 256 to 511 big tiles, e.g. the weight
// gradient of a 512-row out-projection shard, one big tile per CU beats four
// small ones: 0.64 -> 0.50 ms.)
bool use_big_tiles(long long rows, long long cols, long long batch) {
  return ((rows + 255) / 256) * ((cols + 255) / 256) * batch >= 256;
}

// `mode` (FwdMode): every tile, or only those of the mask's uniform or mixed
// 256-channel groups.
template <int BM, int BN, int NW>
int launch_fwd(const uint16_t* X, const uint16_t* W, const uint8_t* mask, uint16_t* out, int T, int M, int Kr,
               int H, hipStream_t s, int mode = kFwdAll) {
  const int tm = (H + BM - 1) / BM, tn = (M + BN - 1) / BN;  // channel tiles x token tiles
  hipLaunchKernelGGL((rowpar_pcr_fwd_kernel<BM, BN, NW>), dim3(tm * tn), dim3(NW * 64), 0, s, X, W, mask, out, T,
                     M, Kr, H, tm, tn, mode);
  return launched();
}

// The forward with the earlier ranks' tiles held in registers (2 <= T <= 8).
template <int BM, int BN, int NW>
int launch_fwd_rb(const uint16_t* X, const uint16_t* W, const uint8_t* mask, uint16_t* out, int T, int M, int Kr,
                  int H, hipStream_t s, int mode = kFwdAll) {
  const int tm = (H + BM - 1) / BM, tn = (M + BN - 1) / BN;
  const dim3 grid(tm * tn), block(NW * 64);
  if (T <= 4)
    hipLaunchKernelGGL((rowpar_pcr_fwd_rb_kernel<BM, BN, NW, 4>), grid, block, 0, s, X, W, mask, out, T, M, Kr, H, tm,
                       tn, mode);
  else if (tm * tn > 2 * kCUs && tm * tn <= 3 * kCUs)  // one round at three per CU, not at two
    hipLaunchKernelGGL((rowpar_pcr_fwd_rb_kernel<BM, BN, NW, 8, 3>), grid, block, 0, s, X, W, mask, out, T, M, Kr, H,
                       tm, tn, mode);
  else
    hipLaunchKernelGGL((rowpar_pcr_fwd_rb_kernel<BM, BN, NW, 8>), grid, block, 0, s, X, W, mask, out, T, M, Kr, H, tm,
                       tn, mode);
  return launched();
}

// G: the backward's reduced gradient; with tile classes (tbits != nullptr)
// only its mixed tiles are per rank, wholly synced ones sit in rank 0's slot
// and wholly local ones are read from dZ.
template <int BM, int BN, int NW>
int launch_dx(const uint16_t* G, const uint16_t* W, uint16_t* dX, int T, int M, int Kr, int H, const uint16_t* dZ,
              const unsigned long long* tbits, hipStream_t s) {
  const int tm = (Kr + BM - 1) / BM, tn = (M + BN - 1) / BN;  // dX column tiles x token tiles
  hipLaunchKernelGGL((pcr_bwd_dx_kernel<BM, BN, NW>), dim3(T * tm * tn), dim3(NW * 64), 0, s, G, W, dX, T, M, Kr,
                     H, tm, tn, dZ, tbits);
  return launched();
}

template <int BM, int BN, int NW>
int launch_dw(const uint16_t* G, const uint16_t* X, uint16_t* dW, int T, int M, int Kr, int H, const uint16_t* dZ,
              const unsigned long long* tbits, hipStream_t s) {
  const int tm = (H + BM - 1) / BM, tn = (Kr + BN - 1) / BN;  // channel tiles x dW row tiles
  hipLaunchKernelGGL((pcr_bwd_dw_kernel<BM, BN, NW>), dim3(T * tm * tn), dim3(NW * 64), 0, s, G, X, dW, T, M, Kr,
                     H, tm, tn, nullptr, 1, (M + kBK - 1) / kBK, dZ, tbits);
  return launched();
}

// Split of dW's token range when its tiles cannot fill the chip: dW_t =
// X_t^T G_t is cut into pieces of at least eight 64-token chunks.  With 64
// to 255 tiles of 256 x 256 those are split into 2-4 pieces, the count that
// best fills whole rounds of 256 workgroups (192 tiles: 4 pieces, 3 full
// rounds); with fewer, 128 x 128 tiles are split until about 256 run.
// splits == 1: no split.
struct DwSplit {
  int splits, kcs;
  bool big;
};
DwSplit dw_split(int T, int M, int Kr, int H) {
  const int nkm = (M + kBK - 1) / kBK;
  DwSplit d{1, nkm, false};
  if (M <= 0 || use_big_tiles(Kr, H, T)) return d;
  const long long big = (long long)((H + 255) / 256) * ((Kr + 255) / 256) * T;
  int sp = 1;
  if (big >= 64) {
    double best = 0.0;
    for (int c = 2; c <= 4 && c <= nkm / 8; ++c) {
      const long long n = big * c, rounds = (n + 255) / 256;
      const double fill = (double)n / (256.0 * (double)rounds);
      if (fill > best + 1e-9) best = fill, sp = c;
    }
    d.big = sp > 1;
  } else {
    const long long tiles = (long long)((H + 127) / 128) * ((Kr + 127) / 128) * T;
    if (tiles >= 256) return d;
    sp = (int)((256 + tiles - 1) / tiles);
    if (sp > nkm / 8) sp = nkm / 8;
  }
  if (sp < 2) return DwSplit{1, nkm, false};
  d.kcs = (nkm + sp - 1) / sp;
  d.splits = (nkm + d.kcs - 1) / d.kcs;  // every piece has at least one chunk
  return d;
}

size_t dw_split_bytes(int T, int M, int Kr, int H) {
  const DwSplit d = dw_split(T, M, Kr, H);
  return d.splits > 1 ? (size_t)d.splits * T * Kr * H * sizeof(float) : 0;
}

// dW through fp32 pieces in `part` (dw_split_bytes of them), then their sum.
int launch_dw_split(const uint16_t* G, const uint16_t* X, uint16_t* dW, int T, int M, int Kr, int H, float* part,
                    const DwSplit& d, const uint16_t* dZ, const unsigned long long* tbits, hipStream_t s) {
  if (d.big) {
    const int tm = (H + 255) / 256, tn = (Kr + 255) / 256;
    hipLaunchKernelGGL((pcr_bwd_dw_kernel<256, 256, kBigTileWaves, true>), dim3(T * d.splits * tm * tn),
                       dim3(kBigTileWaves * 64), 0, s, G, X, dW, T, M, Kr, H, tm, tn, part, d.splits, d.kcs, dZ,
                       tbits);
  } else {
    const int tm = (H + 127) / 128, tn = (Kr + 127) / 128;
    hipLaunchKernelGGL((pcr_bwd_dw_kernel<128, 128, 4, true>), dim3(T * d.splits * tm * tn), dim3(256), 0, s, G, X,
                       dW, T, M, Kr, H, tm, tn, part, d.splits, d.kcs, dZ, tbits);
  }
  if (int st = launched()) return st;
  const long long n4 = (long long)T * Kr * H / 4;
  hipLaunchKernelGGL(dw_split_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, part, dW, d.splits,
                     n4);
  return launched();
}

// Last argument of the reduce kernels: how many row regions consecutive
// workgroups alternate between.  How much the T slices (slice_bytes apart)
// camp on the same HBM channels depends on where the input and the output
// sit in physical memory, which the virtual addresses do not show (the same
// addresses ran at 753 and at 803 us in two processes).  The counts below
// are the ones measured best over twelve placements of Y and out (offsets
// of 0 to 256 MiB and of 4 KiB between them) on [T,16384,4096]:
//   T <= 8, 256 MiB slices (fp32): 16 regions 751-804 us, 2: 764-793,
//          8: 747-882, 4: 770-942, 32: 772-794;
//   T <= 8, 128 MiB slices (bf16): 2 regions 374-384 us, 8: 388-414,
//          16: 390-405;
//   T = 16 (the runtime-T kernel), 128 MiB: 8 regions 887-904 us (16:
//          927-974, 2: 932-998); 256 MiB: 8 regions 1758-1876 us (16:
//          1816-1906, 2: 1829-1907).
// Other spacings: 2 regions for multiples of 16 MiB, else none (the grid
// must divide).  The region count changes no result, only the order in
// which workgroups take the rows.
static uint32_t reduce_groups(const dim3& grid, long long slice_bytes, int T) {
  const long long MiB = 1ll << 20;
  uint32_t g = 1u;
  if (T > 8)
    g = slice_bytes % (128 * MiB) == 0 ? 8u : slice_bytes % (16 * MiB) == 0 ? 2u : 1u;
  else
    g = slice_bytes % (256 * MiB) == 0 ? 16u : slice_bytes % (16 * MiB) == 0 ? 2u : 1u;
  return grid.x % g == 0 ? g : 1u;
}

// Partial channel-reduce of fp32 y[T,M,H] into bf16 o (the split forward's
// second pass).
// (ks contraction slices per rank: y[q][t] at y + (q * T + t) * M * H;
// skip_local: the first pass wrote the wholly local 64-channel groups.)
int launch_reduce_f32_bf16(const float* y, const uint8_t* mask, uint16_t* o, int T, int M, int H, int ks,
                           int skip_local, hipStream_t s) {
  const long long mh = (long long)M * H, ss = (long long)T * mh;
  const uint32_t nvec = (uint32_t)(mh / 4);
  const dim3 grid((nvec + kReduceThreads - 1) / kReduceThreads);
  const uint32_t hv = (uint32_t)(H / 4);
  const uint32_t hf = reduce_groups(grid, mh * 4, T);
  switch (T) {
    case 2: hipLaunchKernelGGL(pcr_reduce_f32_bf16_kernel<2>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, hf, ks, ss, skip_local); break;
    case 4: hipLaunchKernelGGL(pcr_reduce_f32_bf16_kernel<4>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, hf, ks, ss, skip_local); break;
    case 8: hipLaunchKernelGGL(pcr_reduce_f32_bf16_kernel<8>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, hf, ks, ss, skip_local); break;
    case 16: hipLaunchKernelGGL(pcr_reduce_f32_bf16_kernel<16>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, hf, ks, ss, skip_local); break;
    default: hipLaunchKernelGGL(pcr_reduce_f32_bf16_kernel<0>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, hf, ks, ss, skip_local); break;
  }
  return launched();
}

// bf16 partial channel-reduce of y[T,M,H] into o (o == y: in place).  With
// tbits (the backward's G, out of place), wholly local tiles of channels are
// skipped and wholly synced ones written to rank 0's slot only.
int launch_reduce_bf16(const uint16_t* y, const uint8_t* mask, uint16_t* o, int T, int M, int H, hipStream_t s,
                       const unsigned long long* tbits = nullptr) {
  const long long mh = (long long)M * H;
  const uint32_t nvec = (uint32_t)(mh / 8);
  const dim3 grid((nvec + kReduceThreads - 1) / kReduceThreads);
  const int ip = (y == o) ? 1 : 0;
  const uint32_t hv = (uint32_t)(H / 8);
  const uint32_t hf = reduce_groups(grid, mh * 2, T);
  switch (T) {
    case 2: hipLaunchKernelGGL(pcr_reduce_bf16_kernel<2>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip, hf, tbits); break;
    case 4: hipLaunchKernelGGL(pcr_reduce_bf16_kernel<4>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip, hf, tbits); break;
    case 8:
      if (ip) {
        hipLaunchKernelGGL(pcr_reduce_bf16_kernel<8>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip, hf,
                           tbits);
      } else {  // stores regrouped by rank ([8,16384,4096]: 379-381 -> 361-374 us)
        const dim3 g2((nvec + kReduceRunThreads - 1) / kReduceRunThreads);
        hipLaunchKernelGGL(pcr_reduce_bf16_runs8_kernel, g2, dim3(kReduceRunThreads), 0, s, y, mask, o, nvec, hv, mh,
                           reduce_groups(g2, mh * 2, T), tbits);
      }
      break;
    case 16:
      if (ip) {
        hipLaunchKernelGGL(pcr_reduce_bf16_kernel<16>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip,
                           hf, tbits);
      } else {  // stores regrouped by rank ([16,16384,4096]: 780 -> 737 us)
        const dim3 g2((nvec + kReduceRunThreads - 1) / kReduceRunThreads);
        hipLaunchKernelGGL(pcr_reduce_bf16_runs16_kernel, g2, dim3(kReduceRunThreads), 0, s, y, mask, o, nvec, hv, mh,
                           reduce_groups(g2, mh * 2, T), tbits);
      }
      break;
    default: hipLaunchKernelGGL(pcr_reduce_bf16_kernel<0>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip, hf, tbits); break;
  }
  return launched();
}


}  // namespace

extern "C" {

int caat_abi_version(void) { return 1; }

const char* caat_status_string(int status) {
  switch (status) {
    case CAAT_OK: return "ok";
    case CAAT_ERR_NULL: return "null pointer";
    case CAAT_ERR_DIM: return "invalid dimensions (need 1<=T<=64, M>=0, Kr and H positive multiples of 8)";
    case CAAT_ERR_ALIGN: return "misaligned pointer (tensors 16-byte, mask 8-byte)";
    case CAAT_ERR_ALIAS: return "output overlaps an input or another output";
    case CAAT_ERR_DTYPE: return "unknown dtype";
    case CAAT_ERR_WORKSPACE: return "workspace missing or too small";
    case CAAT_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

// Decode-shaped calls: up to kDecChunkedMaxM tokens, taken 32 at a time by
// the weight-streaming kernel (each chunk reads the weights once more; up
// to six chunks that still beats the tiled kernel, which has too few tiles
// to fill the chip at these sizes), and one chunk's fp32 partials [32][H]
// addressable with 32-bit byte offsets.
// Up to kDecMaxH channels, so that the arrival counters (one int per
// 128-channel block) fit a region of fixed size at the head of the
// workspace: a workspace zeroed once stays valid for every later shape.
constexpr int kDecMaxH = 65536;
static bool use_decode(int M, int H) { return M > 0 && M <= kDecChunkedMaxM && H <= kDecMaxH; }

// Arrival counters of the decode kernel: a fixed 2 KiB, whatever H.
constexpr size_t kDecCounterBytes = (size_t)(kDecMaxH / kDecCols) * sizeof(int);
static_assert(kDecCounterBytes % 256 == 0, "partials stay 256-byte aligned");
static size_t decode_counter_bytes(int) { return kDecCounterBytes; }

// Contraction slices per rank for the decode kernel: doubled while the
// workgroups (T * H/128 * ks) stay within one per CU, T * ks <= 8 and every
// wave keeps at least two 32-row stages of each slice.  So T * ks * H is at
// most 32768 when ks > 1, and the sliced partials (ks * T * 32 * H fp32) take
// at most 4 MiB.  Measured on MI355X (M = 1, weights streamed from HBM,
// whole -> sliced, us): T = 1, Kr = 11008, H = 4096: 67.9 -> 20.0 (ks = 8);
// T = 2, Kr = 5504: 38.4 -> 20.1 (4); T = 4, Kr = 2752: 24.2 -> 20.2 (2);
// T = 2, Kr = 2816, H = 2048: 20.8 -> 11.7 (4); T = 4, Kr = 1024, H = 4096:
// 12.1 -> 11.9 (2).  Two workgroups per CU, or one stage per wave, measured
// the same.
constexpr int kDecTargetWG = kCUs;
static int dec_ks(int T, int Kr, int H) {
  const int items = T * ((H + kDecCols - 1) / kDecCols);
  const int ns = (Kr + kDecStage - 1) / kDecStage;
  int ks = 1;
  while (2 * ks <= kDecMaxKs && 2 * ks * T <= 8 && 2 * ks * items <= kDecTargetWG && ns >= 2 * ks * 2 * kDecWaves)
    ks *= 2;
  return ks;
}

// Token counts between decode and full tiles: the rank walk split across
// workgroups, one per (rank, channel block, token block) with the tiles and
// contraction slices of split_plan below, each writing its rank's fp32
// product tile into the workspace (after the decode kernel's counter region,
// which this path leaves alone), then one streaming pass forms the partial
// channel-reduce into out.
// It pays while the fused kernel is short of tiles (of 128 channels x 64
// tokens) for the length of its serial walk, walk = T x ceil(Kr/64) chunks:
// up to 3 x walk + 128 tiles with T <= 8, 2 x walk + 64 with more ranks (the
// second pass reads T ranks' fp32 products), and only up to 128 tiles when
// each rank's contraction is at most two chunks (the fused kernel then holds
// the ranks' tiles in registers).  Measured on MI355X (random S, fused ->
// split, us):
//   T=8  Kr=1376 H=4096 (walk 176): M = 128 / 256 / 512 / 1024 / 1280 / 1536:
//        91 / 164 / 170 / 196 / 220 / 238 -> 37 / 47 / 90 / 165 / 194 / 236
//        (M = 1664: 357 -> 254, past the rule: the fused kernel's second round)
//   T=4  Kr=1376 H=4096 (88): M = 256 / 512 / 768 / 960: 73 / 80 / 82 / 83 -> 32 / 45 / 66 / 77
//   T=8  Kr=704  H=2048 (88): M = 512 / 1024 / 1536 / 1920: 71 / 75 / 85 / 113 -> 31 / 55 / 78 / 100
//   T=8  Kr=512  H=4096 (64): M = 256 / 512 / 640 / 768: 55 / 60 / 67 / 69 -> 26 / 54 / 61 / 72
//   T=8  Kr=384  H=768  (48): M = 1024 / 2304 / 3328: 45 / 50 / 58 -> 24 / 40 / 50
//   T=8  Kr=96   H=768  (16): M = 1024 / 1600: 23 / 23 -> 21 / 29
//   T=16 Kr=688  H=4096 (176): M = 256 / 512 / 960: 178 / 193 / 230 -> 87 / 148 / 242
// Below that the weight-streaming kernel runs (with few ranks in contraction
// slices), up to its 32-token limit with T <= 8; with more ranks (no slices,
// and its exchange grows with T x M) the split takes over at 24 tokens.
// Measured on MI355X, random S, weights streamed from HBM, split ->
// streaming, us: T = 2, Kr = 5504, H = 4096, M = 16 / 32: 40.5 / 40.6 ->
// 21.2 / 24.4; T = 2, Kr = 512: 13.1 / 12.5 -> 9.7 / 9.8; T = 3, Kr = 2000,
// H = 2048: 19.5 / 20.2 -> 13.3 / 16.3; T = 4, Kr = 2752: 25.6 / 26.2 ->
// 21.3 / 25.1; T = 2, Kr = 5504, H = 16384: 65.9 / 68.0 -> 61.8 / 63.4.  The
// split wins by 1-2 us at T = 4 from 20 or 28 tokens with short
// contractions (Kr = 1024, H = 4096, M = 32: 14.1 -> 16.1; Kr = 1408,
// H = 2048: 14.9 -> 16.1).  T = 16, Kr = 688, H = 4096, streaming -> split:
// M = 16 / 24 / 32: 25.1 / 34.4 / 37.3 -> 26.8 / 27.5 / 28.0; T = 8,
// Kr = 1376, M = 24 / 32: 22.7 / 23.5 -> 24.5 / 25.0.
static int split_min_m(int T) { return T <= 8 ? kDecMaxM + 1 : 24; }
static bool use_split(int T, int M, int Kr, int H) {
  const long long tiles = (long long)((H + 127) / 128) * ((M + 63) / 64);
  const long long nk = (Kr + kBK - 1) / kBK, walk = (long long)T * nk;
  const long long limit = nk <= 2 ? 128 : T <= 8 ? 3 * walk + 128 : 2 * walk + 64;
  return T >= 2 && M >= split_min_m(T) && tiles <= limit;
}

// Slices of each rank's contraction in the split forward's 128 x 64 tiles:
// two when those tiles leave at most one workgroup per CU and each rank's
// contraction is long (at least 16 chunks), so that every CU runs two
// workgroups of half the walk; the fp32 products then take twice the
// workspace.  Measured on MI355X (random S, us, 1 -> 2 slices, operands
// resident in the last-level cache): T = 8, Kr = 1376, H = 4096, M = 33 /
// 64: 22.9 / 27.7 -> 22.0 / 24.6; T = 4, M = 64 / 128: 20.8 / 22.0 ->
// 17.9 / 19.1; T = 2, M = 64 / 256: 14.4 / 20.5 -> 12.7 / 20.1.  Slower
// with 512 workgroups (T = 8, M = 96: 24.9 -> 30.9) and with short
// contractions (Kr = 512 or 704, 8 or 11 chunks: +10 to +15%); four slices
// were slower than two everywhere but at T = 4, M = 64 (17.0 us).
constexpr int kMaxSplitKs = 2;
static int split_ks_rule(int T, int M, int Kr, int H) {
  const long long wg = (long long)T * ((H + 127) / 128) * ((M + 63) / 64);
  const int nk = (Kr + kBK - 1) / kBK;
  return wg <= kCUs && nk >= 16 ? 2 : 1;
}

// Tiles of the split forward, and the number of slices each rank's
// contraction is cut into.  256 x 256 tiles (eight waves, half the copy
// bytes per flop) when they fill whole rounds of one workgroup per CU, or one
// round nearly (192 to 256 of them); 128-token tiles once those still give
// two workgroups per CU (at T = 8, H = 4096, M = 256 / 512 / 768: 68 / 100 /
// 138 -> 47 / 90 / 120 us); else 64-token ones (M = 128 there: 36 against
// 38 us).  256 x 256 against 128-channel tiles, same bits (us, operands
// resident in the last-level cache): T = 8, Kr = 1376, H = 4096, M = 512 /
// 1024 (256 / 512 tiles): 73.9 / 141.8 -> 68.7 / 128.6; T = 8, Kr = 704,
// H = 2048, M = 1024 / 1920: 52.5 / 100.2 -> 49.7 / 96.2; T = 8, Kr = 512,
// M = 512: 46.6 -> 43.1; T = 16, Kr = 688, M = 256 / 512: 61.2 / 115.8 ->
// 57.8 / 109.0; 192 and 216 tiles (T = 4, M = 768; T = 8, Kr = 384, H = 768,
// M = 2304): 60.3 / 39.9 -> 53.5 / 36.4.  Slower at 384 tiles (1.5 rounds:
// +4 to +10%) and below 192 (+25 to +60%), and at T = 4, Kr = 1376, M = 960
// (256 tiles): 64.4 -> 66.9.  Only with token tiles at least 3/4 full: at
// T = 16, Kr = 688, M = 64 / 128 (256 tiles, a quarter / half full) they
// took 32.5 / 38.9 us against 28.0 / 34.6 with 128 x 128 tiles.
struct SplitPlan {
  int bm, bn, ks;
};
static SplitPlan split_plan(int T, int M, int Kr, int H) {
  const long long wg128 = (long long)T * ((H + 127) / 128) * ((M + 127) / 128);
  const long long tn256 = (M + 255) / 256, wg256 = (long long)T * ((H + 255) / 256) * tn256;
  const bool full = 4LL * M >= 3LL * 256 * tn256;
  if (full && (wg256 % kCUs == 0 || (wg256 >= 192 && wg256 < kCUs))) return {256, 256, 1};
  if (wg128 >= 512) return {128, 128, 1};
  return {128, 64, split_ks_rule(T, M, Kr, H)};
}

// Workspace of a forward with a mask; `split` = the most contraction slices
// the split path may use, 0 = not at all (the allocation-free entry point
// lowers it, or declines the split, when the fp32 products would not fit the
// library's scratch array).
static size_t fwd_need(int T, int M, int Kr, int H, int split) {
  if (split > 0 && use_split(T, M, Kr, H)) {
    const int ks = std::min(split, split_plan(T, M, Kr, H).ks);
    return kDecCounterBytes + round256((size_t)ks * T * M * H * sizeof(float));
  }
  if (!use_decode(M, H)) return 0;
  return decode_counter_bytes(H) +
         round256((size_t)dec_ks(T, Kr, H) * T * (M < kDecMaxM ? M : kDecMaxM) * H * sizeof(float));
}

size_t caat_rowpar_pcr_fwd_workspace_bytes(int T, int M, int Kr, int H) {
  if (check_dims(T, M, Kr, H) != CAAT_OK) return 0;
  return fwd_need(T, M, Kr, H, kMaxSplitKs);
}

}  // extern "C"

namespace {

// Argument checks of the forward (host only), apart from the workspace.
int fwd_check_args(const uint16_t* X, const uint16_t* W, const uint8_t* mask, const uint16_t* out, int T, int M,
                   int Kr, int H) {
  if (int st = check_dims(T, M, Kr, H)) return st;
  // tensors with no elements (M == 0) may be passed as NULL
  if (!W || (M > 0 && (!X || !out))) return CAAT_ERR_NULL;
  if (!aligned(X, 16) || !aligned(W, 16) || !aligned(out, 16) || !aligned(mask, 8)) return CAAT_ERR_ALIGN;
  const size_t nX = (size_t)T * M * Kr * 2, nW = (size_t)T * Kr * H * 2, nO = (size_t)T * M * H * 2;
  if (M > 0 && (overlap(out, nO, X, nX) || overlap(out, nO, W, nW) || (mask && overlap(out, nO, mask, H))))
    return CAAT_ERR_ALIAS;
  return CAAT_OK;
}

// Kernel launches of a validated forward.  `workspace` starts with the
// decode kernel's arrival counters (kDecCounterBytes, zero on entry); after
// them come the decode kernel's fp32 partials or the split path's fp32
// products (at most `split` contraction slices of them; 0 = no split path).
// Only calls with a mask on those two paths touch it.
int fwd_launch(const uint16_t* X, const uint16_t* W, const uint8_t* mask, uint16_t* out, int T, int M, int Kr,
               int H, void* workspace, hipStream_t s, int split = kMaxSplitKs) {
  if (M == 0) return CAAT_OK;
  if (!mask) workspace = nullptr;  // never touched without synced channels
  if (split > 0 && use_split(T, M, Kr, H)) {
    float* Y = workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kDecCounterBytes) : nullptr;
    const SplitPlan pl = split_plan(T, M, Kr, H);
    const int ks = Y ? std::min(split, pl.ks) : 1;  // bf16 straight to out: whole contractions
    const int tm = (H + pl.bm - 1) / pl.bm, tn = (M + pl.bn - 1) / pl.bn;
    const dim3 grid((unsigned)((long long)T * ks * tm * tn));
    // With whole contractions and H a multiple of 64, the 64-channel groups
    // with no synced channel go straight to out in bf16 and the second pass
    // skips them.
    const uint8_t* lmask = Y && ks == 1 && H % 64 == 0 ? mask : nullptr;
    if (pl.bm == 256)
      hipLaunchKernelGGL((rowpar_pcr_split_kernel<256, 256, kBigTileWaves>), grid, dim3(kBigTileWaves * 64), 0, s, X,
                         W, out, Y, T, M, Kr, H, tm, tn, ks, lmask);
    else if (pl.bn == 128)
      hipLaunchKernelGGL((rowpar_pcr_split_kernel<kSplitBM, 128, kSplitNW>), grid, dim3(kSplitNW * 64), 0, s, X, W,
                         out, Y, T, M, Kr, H, tm, tn, ks, lmask);
    else
      hipLaunchKernelGGL((rowpar_pcr_split_kernel<kSplitBM, 64, kSplitNW>), grid, dim3(kSplitNW * 64), 0, s, X, W,
                         out, Y, T, M, Kr, H, tm, tn, ks, lmask);
    if (int st = launched()) return st;
    return Y ? launch_reduce_f32_bf16(Y, mask, out, T, M, H, ks, lmask != nullptr, s) : CAAT_OK;
  }
  if (use_decode(M, H)) {
    // workspace: the per-block arrival counters, then the fp32 partials
    int* arrivals = static_cast<int*>(workspace);
    float* partial =
        workspace ? reinterpret_cast<float*>(static_cast<char*>(workspace) + decode_counter_bytes(H)) : nullptr;
    const int ks = partial ? dec_ks(T, Kr, H) : 1;  // no workspace (no mask): whole contractions
    const dim3 grid(((H + kDecCols - 1) / kDecCols) * T * ks);
    const long long xs = (long long)M * Kr, os = (long long)M * H;  // rank strides of X and out
    // Chunks run one after another on the stream and share the workspace;
    // each launch leaves the arrival counters at zero for the next.
    for (int m0 = 0; m0 < M; m0 += kDecMaxM) {
      const int mc = M - m0 < kDecMaxM ? M - m0 : kDecMaxM;
      const uint16_t* Xc = X + (long long)m0 * Kr;
      uint16_t* oc = out + (long long)m0 * H;
      if (mc <= 16 && ks == 1)
        hipLaunchKernelGGL((rowpar_pcr_decode_kernel<1, false>), grid, dim3(kDecThreads), 0, s, Xc, W, mask, oc,
                           partial, arrivals, T, mc, Kr, H, xs, os, ks);
      else if (mc <= 16)
        hipLaunchKernelGGL((rowpar_pcr_decode_kernel<1, true>), grid, dim3(kDecThreads), 0, s, Xc, W, mask, oc,
                           partial, arrivals, T, mc, Kr, H, xs, os, ks);
      else if (ks == 1)
        hipLaunchKernelGGL((rowpar_pcr_decode_kernel<2, false>), grid, dim3(kDecThreads), 0, s, Xc, W, mask, oc,
                           partial, arrivals, T, mc, Kr, H, xs, os, ks);
      else
        hipLaunchKernelGGL((rowpar_pcr_decode_kernel<2, true>), grid, dim3(kDecThreads), 0, s, Xc, W, mask, oc,
                           partial, arrivals, T, mc, Kr, H, xs, os, ks);
      if (int st = launched()) return st;
    }
    return CAAT_OK;
  }
  // Fewer than 512 tiles of 128 x 128 (two per CU): 64-token tiles give
  // twice as many workgroups (each walks all T ranks, so the tile count is
  // what fills the chip), up to three resident per CU.  Measured with the
  // same bits: 130M down-proj (384 tiles) 100 -> 91 us, out-proj 74 -> 68 us,
  // 7B down-proj at M = 1024 (256 tiles) 179 -> 154 us; at 512-1023 tiles the
  // 64-token tiles lose (M = 2048: 243 -> 321 us).
  // 256 x 256 tiles from 160 of them (5/8 of the CUs; the products need
  // 256): measured, 128 x 128 -> 256 x 256 tiles, us: T = 8, Kr = 1376,
  // H = 4096, M = 2560 / 3072 / 3584 / 3840 (160 / 192 / 224 / 240 tiles):
  // 391 / 394 / 432 / 444 -> 345 / 345 / 370 / 386; T = 4, Kr = 2752,
  // M = 2560 / 3584: 309 / 348 -> 259 / 301; T = 16, Kr = 688, M = 3584:
  // 566 -> 500; Kr = 512 or 704: 2-7% faster.  With 128 of them they lose
  // (T = 8, Kr = 1376, M = 2048: 235 -> 317).
  const bool big = (long long)((M + 255) / 256) * ((H + 255) / 256) >= kFwdBigTiles;
  const bool small = !big && (long long)((H + 127) / 128) * ((M + 127) / 128) < 512;
  // The earlier ranks' tiles held in registers, for every tile: with T <= 4
  // (three workgroups per CU still fit) and, at two per CU, for contractions
  // of at most two chunks per rank.  Measured, same bits, M = 8192, H = 768,
  // random S: Kr = 384, T = 2 22.5 -> 18.8 us, T = 4 45.3 -> 34.0 us;
  // Kr = 96, T = 8 67.3 -> 47 us.
  if (small && mask != nullptr && T >= 2 && (T <= 4 || (T <= 8 && Kr <= 2 * kBK)))
    return launch_fwd_rb<128, 64, 4>(X, W, mask, out, T, M, Kr, H, s);
  // With short contractions (at most six chunks per rank) and 2 <= T <= 8,
  // the register-queue kernel takes the mask's mixed 256-channel groups (an
  // 8-channel chunk with synced and local channels: the tiled kernels write
  // those lines twice) and the tiled kernel the uniform ones, in two
  // launches.  Measured at T = 8 with a random S (every group mixed), tiled
  // -> register queue, us: Kr = 128, H = 2048, M = 8192 / 32768: 185 / 596
  // -> 108 / 390; Kr = 256, H = 2048, M = 2048 / 8192 / 32768: 63 / 208 /
  // 640 -> 42 / 145 / 581; Kr = 256, H = 4096, M = 2048 / 8192 / 16384: 98 /
  // 396 / 679 -> 73 / 302 / 586; Kr = 192 / 384, H = 768, M = 16384: 138 /
  // 172 -> 91 / 136.  With longer contractions the queue kernel loses at
  // large M (Kr = 512, H = 4096, M = 16384: 831 -> 948; Kr = 704, H = 2048,
  // M = 32768: 1091 -> 1566), and with a contiguous S (uniform groups) it
  // loses too, so those keep the tiled kernels.  Where the 128 x 64 tiles
  // run anyway, contractions of up to twelve chunks still gain (Kr = 512 /
  // 704, H = 2048, M = 2048: 81 / 102 -> 60 / 81 us).
  const int nkr = (Kr + kBK - 1) / kBK;
  const bool dual = mask != nullptr && T >= 2 && T <= 8 && (nkr <= 6 || (small && nkr <= 12));
  const int mode = dual ? kFwdUniform : kFwdAll;
  int st;
  if (big)
    st = launch_fwd<256, 256, kBigTileWaves>(X, W, mask, out, T, M, Kr, H, s, mode);
  else if (small)
    st = launch_fwd<128, 64, 4>(X, W, mask, out, T, M, Kr, H, s, mode);
  else
    st = launch_fwd<128, 128, 4>(X, W, mask, out, T, M, Kr, H, s, mode);
  if (st != CAAT_OK || !dual) return st;
  return launch_fwd_rb<128, 64, 4>(X, W, mask, out, T, M, Kr, H, s, kFwdMixed);
}

// Shared by the row-parallel forward (mask = S) and the column-parallel
// forward (mask == nullptr: nothing synced, no workspace used).
int fwd_impl(const uint16_t* X, const uint16_t* W, const uint8_t* mask, uint16_t* out, int T, int M, int Kr, int H,
             void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = fwd_check_args(X, W, mask, out, T, M, Kr, H)) return st;
  const size_t need = mask ? caat_rowpar_pcr_fwd_workspace_bytes(T, M, Kr, H) : 0;
  if (need > 0) {
    const size_t nX = (size_t)T * M * Kr * 2, nW = (size_t)T * Kr * H * 2, nO = (size_t)T * M * H * 2;
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return CAAT_ERR_WORKSPACE;
    if (overlap(workspace, need, out, nO) || overlap(workspace, need, X, nX) || overlap(workspace, need, W, nW) ||
        overlap(workspace, need, mask, H))
      return CAAT_ERR_ALIAS;
  }
  return fwd_launch(X, W, mask, out, T, M, Kr, H, workspace, reinterpret_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" {

int caat_rowpar_pcr_fwd(const uint16_t* X, const uint16_t* W, const uint8_t* mask, uint16_t* out, int T, int M,
                        int Kr, int H, void* workspace, size_t workspace_bytes, void* stream) {
  if (!mask) return CAAT_ERR_NULL;
  return fwd_impl(X, W, mask, out, T, M, Kr, H, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// ---- forward without a caller workspace -----------------------------------
// Library-owned scratch for the decode kernel's arrival counters and fp32
// partials, or the split path's fp32 products, one copy per GPU (each device holds its own instance of this
// array, at its own address, until the process ends; it starts zeroed).  In
// host code the array's name is only a host-side stand-in: kernels get the
// device address that hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = (size_t)CAAT_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];  // device address of `scratch` per device (null: not looked up yet)

// Device address of the current device's scratch, looked up once per device.
int scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return CAAT_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return CAAT_ERR_LAUNCH;
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return CAAT_OK;
}

}  // namespace

extern "C" {

int caat_rowpar_pcr_fwd_noalloc(const uint16_t* X, const uint16_t* W, const uint8_t* mask, uint16_t* out, int T,
                                int M, int Kr, int H, void* stream) {
  if (!mask) return CAAT_ERR_NULL;
  if (int st = fwd_check_args(X, W, mask, out, T, M, Kr, H)) return st;
  // The split path's fp32 products may not fit the scratch array: then
  // fewer contraction slices, or, if even one does not fit, the tiled or
  // chunked decode path (no scratch, or a chunk's).
  int split = kMaxSplitKs;
  while (split > 0 && fwd_need(T, M, Kr, H, split) > kScratchBytes) split /= 2;
  const size_t need = fwd_need(T, M, Kr, H, split);
  if (need > kScratchBytes) return CAAT_ERR_WORKSPACE;
  if (M == 0) return CAAT_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* ws = nullptr;
  if (need > 0) {
    if (int st = scratch_ptr(&ws)) return st;
    // The arrival counters must start at zero: clear them with a small fill
    // kernel (not a memset, so that the call can be captured in a graph).
    const long long nc = (long long)(kDecCounterBytes / sizeof(uint32_t));
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((nc + 255) / 256)), dim3(256), 0, s,
                       static_cast<uint32_t*>(ws), nc, 0u);
    if (int st = launched()) return st;
  }
  return fwd_launch(X, W, mask, out, T, M, Kr, H, ws, s, split);
}

int caat_colpar_fwd(const uint16_t* A, const uint16_t* W, uint16_t* U, int T, int M, int K, int N, void* stream) {
  return fwd_impl(A, W, nullptr, U, T, M, K, N, nullptr, 0, stream);
}

// The backward's tile classes of channels (two 64-bit masks), after G.
constexpr size_t kClassBytes = 256;

size_t caat_pcr_bwd_workspace_bytes(int T, int M, int Kr, int H) {
  if (check_dims(T, M, Kr, H) != CAAT_OK || M == 0) return 0;
  // G_t for every rank (bf16), the 256-byte tile-class area, then dW's fp32
  // token-range pieces when dW is split
  return round256((size_t)T * M * H * 2) + kClassBytes + dw_split_bytes(T, M, Kr, H);
}

}  // extern "C"

namespace {

// Shared by the row-parallel backward (mask = S: G = the partial
// channel-reduce of dZ, materialised in the workspace) and the
// column-parallel backward (mask == nullptr: G = dZ itself, no workspace).
int bwd_impl(const uint16_t* dZ, const uint16_t* X, const uint16_t* W, const uint8_t* mask, uint16_t* dX,
             uint16_t* dW, int T, int M, int Kr, int H, void* workspace, size_t workspace_bytes, void* stream) {
  if (int st = check_dims(T, M, Kr, H)) return st;
  // dZ and X have no elements when M == 0 and may then be NULL
  if ((M > 0 && !dZ) || (dX && !W) || (M > 0 && dW && !X)) return CAAT_ERR_NULL;
  if (!aligned(dZ, 16) || (X && !aligned(X, 16)) || (W && !aligned(W, 16)) || (dX && !aligned(dX, 16)) ||
      (dW && !aligned(dW, 16)) || !aligned(mask, 8))
    return CAAT_ERR_ALIGN;
  const size_t nX = (size_t)T * M * Kr * 2, nW = (size_t)T * Kr * H * 2, nZ = (size_t)T * M * H * 2;
  const void* ins[4] = {dZ, X, W, mask};  // a NULL entry is skipped
  const size_t nin[4] = {nZ, nX, nW, (size_t)H};
  for (int i = 0; i < 4; ++i) {
    if (!ins[i]) continue;
    if (dX && overlap(dX, nX, ins[i], nin[i])) return CAAT_ERR_ALIAS;
    if (dW && overlap(dW, nW, ins[i], nin[i])) return CAAT_ERR_ALIAS;
  }
  if (dX && dW && overlap(dX, nX, dW, nW)) return CAAT_ERR_ALIAS;
  const size_t need = mask ? caat_pcr_bwd_workspace_bytes(T, M, Kr, H) : 0;
  if (need > 0 && (dX || dW)) {
    if (!workspace || workspace_bytes < need || !aligned(workspace, 16)) return CAAT_ERR_WORKSPACE;
    for (int i = 0; i < 4; ++i)
      if (ins[i] && overlap(workspace, need, ins[i], nin[i])) return CAAT_ERR_ALIAS;
    if ((dX && overlap(workspace, need, dX, nX)) || (dW && overlap(workspace, need, dW, nW))) return CAAT_ERR_ALIAS;
  }
  if (!dX && !dW) return CAAT_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (M == 0) {  // no tokens: dX is empty and dW = X^T G is the zero matrix
    if (dW) {
      const long long n = (long long)T * Kr * H / 2;  // u32 words of bf16 zeros
      hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                         reinterpret_cast<uint32_t*>(dW), n, 0u);
      return launched();
    }
    return CAAT_OK;
  }
  // G_t = the partial channel-reduce of dZ, into the workspace; with nothing
  // synced G is dZ.  Up to 64 tiles of 256 channels (H <= 16384) are first
  // classified: G is then written only for mixed tiles (every rank) and
  // wholly synced ones (rank 0's slot, the one sum); the products read a
  // wholly local tile straight from dZ.  Same values either way.
  const uint16_t* G = dZ;
  const unsigned long long* tbits = nullptr;
  const size_t g_bytes = round256((size_t)T * M * H * 2);
  if (mask) {
    uint16_t* Gw = reinterpret_cast<uint16_t*>(workspace);
    if (H <= kClassCols * kMaxClassTiles) {
      unsigned long long* tb = reinterpret_cast<unsigned long long*>(static_cast<char*>(workspace) + g_bytes);
      hipLaunchKernelGGL(pcr_tile_class_kernel, dim3(1), dim3(64), 0, s, mask, H, tb);
      if (int st = launched()) return st;
      tbits = tb;
    }
    if (int st = launch_reduce_bf16(dZ, mask, Gw, T, M, H, s, tbits)) return st;
    G = Gw;
  }
  if (dX) {
    // (Kr < 256 fills under half of a 256-row tile: the 128-row tiles win
    // there, e.g. Kr = 96, T = 8, M = 8192: backward 94.6 -> 89.3 us; at
    // Kr = 384 and 704 the big tiles stay faster)
    const int st = use_big_tiles(M, Kr, T) && Kr >= 256
                       ? launch_dx<256, 256, kBigTileWaves>(G, W, dX, T, M, Kr, H, dZ, tbits, s)
                       : launch_dx<128, 128, 4>(G, W, dX, T, M, Kr, H, dZ, tbits, s);
    if (st) return st;
  }
  if (dW) {
    const DwSplit d = dw_split(T, M, Kr, H);
    int st;
    if (mask && d.splits > 1)  // the pieces live in the workspace, after G and the tile classes
      st = launch_dw_split(G, X, dW, T, M, Kr, H,
                           reinterpret_cast<float*>(static_cast<char*>(workspace) + g_bytes + kClassBytes), d, dZ,
                           tbits, s);
    else
      st = use_big_tiles(Kr, H, T) ? launch_dw<256, 256, kBigTileWaves>(G, X, dW, T, M, Kr, H, dZ, tbits, s)
                                   : launch_dw<128, 128, 4>(G, X, dW, T, M, Kr, H, dZ, tbits, s);
    if (st) return st;
  }
  return CAAT_OK;
}

}  // namespace

extern "C" {

int caat_pcr_bwd(const uint16_t* dZ, const uint16_t* X, const uint16_t* W, const uint8_t* mask, uint16_t* dX,
                 uint16_t* dW, int T, int M, int Kr, int H, void* workspace, size_t workspace_bytes, void* stream) {
  if (!mask) return CAAT_ERR_NULL;
  return bwd_impl(dZ, X, W, mask, dX, dW, T, M, Kr, H, workspace, workspace_bytes, stream);
}

int caat_colpar_bwd(const uint16_t* dU, const uint16_t* A, const uint16_t* W, uint16_t* dA, uint16_t* dW, int T,
                    int M, int K, int N, void* stream) {
  return bwd_impl(dU, A, W, nullptr, dA, dW, T, M, K, N, nullptr, 0, stream);
}

int caat_partial_channel_reduce(const void* Y, const uint8_t* mask, void* out, int T, int M, int H, int dtype,
                                void* stream) {
  if (dtype != CAAT_F32 && dtype != CAAT_BF16) return CAAT_ERR_DTYPE;
  if (T < 1 || T > kMaxT || M < 0 || H < 8 || H % 8 != 0) return CAAT_ERR_DIM;
  if (!mask || (M > 0 && (!Y || !out))) return CAAT_ERR_NULL;
  if ((long long)T * M * (long long)H > (1LL << 40)) return CAAT_ERR_DIM;
  // one rank's slice below 2^30 elements, as for every call: the kernels
  // count its 16-byte vectors in 32 bits
  if ((long long)M * H >= (1LL << 30)) return CAAT_ERR_DIM;
  if (!aligned(Y, 16) || !aligned(out, 16) || !aligned(mask, 8)) return CAAT_ERR_ALIGN;
  const size_t esz = dtype == CAAT_F32 ? 4 : 2;
  const size_t n = (size_t)T * M * H * esz;
  const bool inplace = (Y == out);
  if (!inplace && overlap(Y, n, out, n)) return CAAT_ERR_ALIAS;
  if (overlap(out, n, mask, H)) return CAAT_ERR_ALIAS;
  if (M == 0) return CAAT_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const long long mh = (long long)M * H;
  if (dtype == CAAT_F32) {
    const uint32_t nvec = (uint32_t)(mh / 4);
    const dim3 grid((nvec + kReduceThreads - 1) / kReduceThreads);
    const float* y = static_cast<const float*>(Y);
    float* o = static_cast<float*>(out);
    const int ip = inplace ? 1 : 0;
    const uint32_t hv = (uint32_t)(H / 4);
    const uint32_t hf = reduce_groups(grid, mh * 4, T);
    switch (T) {
      case 1: hipLaunchKernelGGL(pcr_reduce_f32_kernel<1>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip, hf); break;
      case 2: hipLaunchKernelGGL(pcr_reduce_f32_kernel<2>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip, hf); break;
      case 4: hipLaunchKernelGGL(pcr_reduce_f32_kernel<4>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip, hf); break;
      case 8:
        if (ip) {
          hipLaunchKernelGGL(pcr_reduce_f32_kernel<8>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip, hf);
        } else {  // stores regrouped by rank ([8,16384,4096] over five placements: 742-794 -> 731-767 us)
          const dim3 g2((nvec + kReduceRunThreads - 1) / kReduceRunThreads);
          hipLaunchKernelGGL(pcr_reduce_f32_runs8_kernel, g2, dim3(kReduceRunThreads), 0, s, y, mask, o, nvec, hv, mh,
                             reduce_groups(g2, mh * 4, T));
        }
        break;
      case 16: hipLaunchKernelGGL(pcr_reduce_f32_kernel<16>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip, hf); break;
      default: hipLaunchKernelGGL(pcr_reduce_f32_kernel<0>, grid, dim3(kReduceThreads), 0, s, y, mask, o, T, nvec, hv, mh, ip, hf); break;
    }
  } else {
    return launch_reduce_bf16(static_cast<const uint16_t*>(Y), mask, static_cast<uint16_t*>(out), T, M, H, s);
  }
  return launched();
}

int caat_residual_rmsnorm(const uint16_t* Z, const uint16_t* R, const uint16_t* gamma, uint16_t* Rout, uint16_t* N,
                          int T, int M, int H, float eps, void* stream) {
  if (T < 1 || T > kMaxT || M < 0 || H < 8 || H % 8 != 0 || H > 8 * kNormThreads * kNormMaxVecs) return CAAT_ERR_DIM;
  if ((long long)T * M >= (1LL << 31)) return CAAT_ERR_DIM;
  if (!(eps >= 0.0f) || eps > 1e30f) return CAAT_ERR_DIM;  // also rejects NaN
  if (!gamma || (M > 0 && (!Z || !R || !Rout || !N))) return CAAT_ERR_NULL;
  if (!aligned(Z, 16) || !aligned(R, 16) || !aligned(gamma, 16) || !aligned(Rout, 16) || !aligned(N, 16))
    return CAAT_ERR_ALIGN;
  const size_t n = (size_t)T * M * H * 2, ng = (size_t)H * 2;
  if (M > 0) {
    if (Rout != R && (overlap(Rout, n, R, n) || overlap(Rout, n, Z, n) || overlap(Rout, n, gamma, ng)))
      return CAAT_ERR_ALIAS;
    if (Rout == R && (overlap(R, n, Z, n) || overlap(R, n, gamma, ng))) return CAAT_ERR_ALIAS;
    if (overlap(N, n, Z, n) || overlap(N, n, R, n) || overlap(N, n, Rout, n) || overlap(N, n, gamma, ng))
      return CAAT_ERR_ALIAS;
  }
  if (M == 0) return CAAT_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)((long long)T * M));
  const int hv = H / 8;
  if (hv <= kNormThreads)
    hipLaunchKernelGGL(pcr_residual_rmsnorm_kernel<1>, grid, dim3(kNormThreads), 0, s, Z, R, gamma, Rout, N, H, eps);
  else if (hv <= 2 * kNormThreads)
    hipLaunchKernelGGL(pcr_residual_rmsnorm_kernel<2>, grid, dim3(kNormThreads), 0, s, Z, R, gamma, Rout, N, H, eps);
  else
    hipLaunchKernelGGL(pcr_residual_rmsnorm_kernel<4>, grid, dim3(kNormThreads), 0, s, Z, R, gamma, Rout, N, H, eps);
  return launched();
}


int caat_partial_channel_reduce_residual_rmsnorm(const uint16_t* Y, const uint8_t* mask, const uint16_t* R,
                                                  const uint16_t* gamma, uint16_t* Rout, uint16_t* N, int T, int M,
                                                  int H, float eps, void* stream) {
  if (T < 1 || T > kMaxT || M < 0 || H < 8 || H % 8 != 0 || H > 8 * kNormThreads * kNormMaxVecs) return CAAT_ERR_DIM;
  if ((long long)M * H >= (1LL << 30)) return CAAT_ERR_DIM;
  if (!(eps >= 0.0f) || eps > 1e30f) return CAAT_ERR_DIM;  // also rejects NaN
  if (!mask || !gamma || (M > 0 && (!Y || !R || !Rout || !N))) return CAAT_ERR_NULL;
  if (!aligned(Y, 16) || !aligned(R, 16) || !aligned(gamma, 16) || !aligned(Rout, 16) || !aligned(N, 16) ||
      !aligned(mask, 8))
    return CAAT_ERR_ALIGN;
  const size_t n = (size_t)T * M * H * 2, ng = (size_t)H * 2;
  if (M > 0) {
    const void* ins[3] = {Y, gamma, mask};
    const size_t nin[3] = {n, ng, (size_t)H};
    for (int i = 0; i < 3; ++i)
      if (overlap(Rout, n, ins[i], nin[i]) || overlap(N, n, ins[i], nin[i])) return CAAT_ERR_ALIAS;
    if (overlap(R, n, Y, n)) return CAAT_ERR_ALIAS;
    if (Rout != R && overlap(Rout, n, R, n)) return CAAT_ERR_ALIAS;
    if (overlap(N, n, R, n) || overlap(N, n, Rout, n)) return CAAT_ERR_ALIAS;
  }
  if (M == 0) return CAAT_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid((unsigned)M), block(kNormThreads);
  const long long mh = (long long)M * H;
  const int hv = H / 8;
  const int kv = hv <= kNormThreads ? 1 : hv <= 2 * kNormThreads ? 2 : 4;
  // The T rank slices camp on HBM channels as in the reduce.  With T <= 8
  // the reduce's region count (2 at 128 MiB slices: [8,16384,4096], 795-805
  // -> 780-794 us, same bits; 8 regions: 891-894); plain order otherwise.
  const uint32_t groups = T <= 8 ? reduce_groups(grid, mh * 2, T) : 1u;
#define CAAT_RRN(KV, TC) \
  hipLaunchKernelGGL((pcr_reduce_residual_rmsnorm_kernel<KV, TC>), grid, block, 0, s, Y, mask, R, gamma, Rout, N, T, H, mh, eps, groups)
  if (kv == 1) {
    switch (T) {
      case 1: CAAT_RRN(1, 1); break;
      case 2: CAAT_RRN(1, 2); break;
      case 4: CAAT_RRN(1, 4); break;
      case 8: CAAT_RRN(1, 8); break;
      default: CAAT_RRN(1, 0); break;
    }
  } else if (kv == 2) {
    switch (T) {
      case 1: CAAT_RRN(2, 1); break;
      case 2: CAAT_RRN(2, 2); break;
      case 4: CAAT_RRN(2, 4); break;
      case 8: CAAT_RRN(2, 8); break;
      default: CAAT_RRN(2, 0); break;
    }
  } else {
    CAAT_RRN(4, 0);
  }
#undef CAAT_RRN
  return launched();
}

}  // extern "C"
