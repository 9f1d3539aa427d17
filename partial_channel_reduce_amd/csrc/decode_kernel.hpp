// Decode-shaped forward (M <= 32 tokens): the same result as the fused
// forward, organised for weight streaming.  With so few tokens the layer reads
// ~T*Kr*H*2 bytes of weights once and does almost no arithmetic per byte, so
// it runs as one kernel laid out for HBM streaming:
//
//   rowpar_pcr_decode_kernel: one workgroup per (rank t, 128-channel block),
//     so every weight row piece it reads is 256 contiguous bytes.  Its 8 waves
//     split the contraction (interleaved 32-row stages); each keeps two
//     32-row x 128-channel weight stages loading into registers, writes each
//     stage to its own LDS slot and feeds it to 16x16x32 bf16 MFMAs through
//     gfx950's LDS transpose read; X_t's token rows are loaded straight in the
//     MFMA operand layout.  (Plain loads into registers stream faster here
//     than copies straight into LDS; with the MFMAs removed the kernel is no
//     faster: it is bound by the weight stream.)  The waves' partial sums are
//     added in wave order through LDS.  A channel block with no synced channel
//     is written straight to out[t]; otherwise each workgroup leaves its fp32
//     values in the workspace, and the last of the T workgroups of the block
//     to finish (an arrival counter per block, in the workspace) adds the
//     synced values in ascending rank order and writes every rank's output
//     (the one bf16 sum on synced channels, the rank's own value elsewhere)
//     with whole 8-byte stores.
//   With few ranks or channel blocks (T * H/128 workgroups would leave CUs
//     idle) each rank's contraction is cut into ks slices of whole 32-row
//     stages, one workgroup each (T * ks <= 8).  Every block then goes
//     through the exchange: the last of its T * ks workgroups adds each
//     rank's slices in slice order, then the synced channels over the ranks
//     in ascending order.
#pragma once

#include "gemm_core.hpp"

namespace caat {

constexpr int kDecMaxM = 32;     // two 16-row MFMA blocks per launch
constexpr int kDecMaxKs = 8;     // contraction slices per rank: T * ks <= 8
constexpr int kDecChunkedMaxM = 192;  // larger M up to this: one launch per 32-token chunk
constexpr int kDecCols = 128;    // channels per workgroup: 256 bytes of each weight row
constexpr int kDecWaves = 8;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecStage = 32;    // contraction rows per stage (one MFMA k-step)
constexpr int kDecLpr = kDecCols / 8;       // lanes per weight row piece (16 bytes each)
constexpr int kDecRpi = 64 / kDecLpr;       // weight rows per load instruction
constexpr int kDecLoads = kDecStage / kDecRpi;  // weight loads per stage

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// LDS stage layout [32 k][128 channels], 256-byte rows (one pass over the 64
// banks each); 16-byte chunks XOR swizzled by 2*(k%4) + 8*((k/8)%2): a
// transpose read serves 32 lanes at a time, k-rows {k..k+3} and {k+8..k+11}
// of one 16-channel block, which this spreads over all 64 banks.
__device__ __forceinline__ int dec_off(int k, int ch) {
  return k * kDecCols + (((ch >> 3) ^ (((k & 3) << 1) | (((k >> 3) & 1) << 3))) << 3) + (ch & 7);
}

// NB: MFMA row blocks of 16 tokens, 1 (M <= 16) or 2.  The M token rows of
// rank t start at X + t * xs and out + t * os (xs = M * Kr and os = M * H
// for a whole call; larger when the call is one 32-token chunk of a bigger
// batch, X and out then pointing at the chunk's first row).  SL: the
// contraction may come in ks > 1 slices (without it ks is taken as 1 and the
// slice arithmetic compiles away).
template <int NB, bool SL>
__global__ void __launch_bounds__(kDecThreads)
rowpar_pcr_decode_kernel(const uint16_t* __restrict__ X, const uint16_t* __restrict__ W,
                         const uint8_t* __restrict__ mask, uint16_t* __restrict__ out,
                         float* __restrict__ partial, int* __restrict__ arrivals, int T, int M, int Kr,
                         int H, long long xs, long long os, int ks_arg) {
  const int ks = SL ? ks_arg : 1;
  constexpr int D = 2;                      // stages held in registers: one being used, one loading
  constexpr int SE = kDecStage * kDecCols;  // W elements per stage (4 KiB)
  constexpr int SLOT = SE;                  // one LDS slot per wave
  constexpr int RR = 16 * NB;               // token rows of the fp32 reduction area
  constexpr int LDS = kDecWaves * SLOT > kDecWaves * RR * kDecCols * 2
                          ? kDecWaves * SLOT
                          : kDecWaves * RR * kDecCols * 2;  // slots, or the fp32 reduction area
  __shared__ __attribute__((aligned(16))) uint16_t lds[LDS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nb = (H + kDecCols - 1) / kDecCols;
  // Each XCD takes a contiguous range of (rank, channel block, slice) items,
  // so with T = 8 every XCD serves one rank and its L2 reads that rank's
  // tokens once (numbered rank-major, each rank's blocks would be spread over
  // all eight).
  const int lin = xcd_remap(blockIdx.x, gridDim.x);
  const int per = nb * ks;
  const int t = lin / per;
  const int blk = (lin - t * per) / ks, sl = lin - t * per - blk * ks;
  const int n0 = blk * kDecCols;
  const long long MK = (long long)M * Kr, KH = (long long)Kr * H, MH = (long long)M * H;

  // This workgroup's slice: 32-row stages [s_lo, s_hi) of the rank's
  // contraction; this wave's share of it: stages s_lo + wave, s_lo + wave + 8,
  // ... (the workgroup's waves read adjacent row groups together).
  const int ns_all = (Kr + kDecStage - 1) / kDecStage;
  const int s_lo = sl * ns_all / ks, s_hi = (sl + 1) * ns_all / ks;
  const int nst = (s_hi - s_lo - wave + kDecWaves - 1) / kDecWaves;

  // Operands are loaded into registers D-1 stages ahead (plain buffer loads:
  // the compiler tracks them and waits exactly).  Per lane and stage: 8
  // weight pieces (k-row lane/16 + 4i, 16-byte chunk lane%16), written to this
  // wave's LDS slot for the transposing reads, and NB token pieces loaded
  // straight in the MFMA A-fragment layout (token row lane%16 + 16b, 8-k
  // chunk lane/16).  Weight rows past Kr, token rows past M and X columns
  // past Kr read as zero (out of the buffer's range).
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(W + t * KH, (uint32_t)(KH * 2));
  const uint32_t xbytes = (uint32_t)(MK * 2);
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(X + t * xs, xbytes);
  const int wr = lane / kDecLpr, wc = lane % kDecLpr;
  const int wvoff = (wr * H + wc * 8) * 2;
  const int xr = lane & 15, xc = lane >> 4;  // A-fragment layout: token row, 8-k chunk
  struct Stage {
    u32x4 w[kDecLoads];
    u32x4 x[NB];
  };
  // Stages past this wave's last one are loaded too, wholly out of range (no
  // memory traffic, zeros): every load is unconditional, which lets the
  // compiler count outstanding loads exactly across the unrolled loop.
  const int wend = (int)(KH * 2);
  constexpr int kNt = 1 << 1;  // weights are read once: non-temporal (streaming) loads
  auto load = [&](int st, Stage& S) {
    const bool live = st < nst;
    const int k0 = (s_lo + st * kDecWaves + wave) * kDecStage;
#pragma unroll
    for (int i = 0; i < kDecLoads; ++i)
      S.w[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     wrs, wvoff, __builtin_amdgcn_readfirstlane(
                               live ? (int)(((uint32_t)(k0 + kDecRpi * i) * (uint32_t)H + (uint32_t)n0) * 2u) : wend), kNt));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int m = xr + 16 * b;
      const bool ok = live && m < M && k0 + xc * 8 < Kr;
      const int voff = ok ? (m * Kr + k0 + xc * 8) * 2 : (int)xbytes;
      S.x[b] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs, voff, 0, 0));
    }
  };
  uint16_t* slot = lds + wave * SLOT;

  constexpr int NJ = kDecCols / 16;  // 16-channel MFMA column blocks
  f32x4_t acc[NB][NJ];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[b][j][e] = 0.f;

  // tr-read addressing (16x16x32 B operand): lane 4s+u of 16-lane group g
  // names k-row 8g+4h+s and channels 4u..4u+3 of a 16-channel block.
  const int g = lane >> 4, s4 = (lane & 15) >> 2, u4 = lane & 3;
  auto use = [&](const Stage& S) {
#pragma unroll
    for (int i = 0; i < kDecLoads; ++i) st16(slot + dec_off(wr + kDecRpi * i, wc * 8), S.w[i]);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's writes land before its reads
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      u32x4 bv;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int row = 8 * g + 4 * h + s4;
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(slot + dec_off(row, j * 16 + 4 * u4)));
        const u32x2 w2 = __builtin_bit_cast(u32x2, v);
        bv[2 * h] = w2[0];
        bv[2 * h + 1] = w2[1];
      }
#pragma unroll
      for (int bb = 0; bb < NB; ++bb)
        acc[bb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(S.x[bb]), as_bf16x8(bv), acc[bb][j], 0, 0, 0);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the slot is rewritten
  };

  // Stage st lives in register set st % D; the loop is unrolled D times so
  // every set is named statically (a copy would wait on its loads).  The
  // stage count is padded up to a multiple of D with all-zero stages, so the
  // loop has no early exits.
  Stage r[D];
#pragma unroll
  for (int j = 0; j < D - 1; ++j) load(j, r[j]);
  for (int st = 0; st < nst; st += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      load(st + j + D - 1, r[(j + D - 1) % D]);
      use(r[j]);
    }
  }
  __syncthreads();

  // Add the waves' partial products in wave order.  Accumulator layout
  // (16x16): channel 16j + lane%16, token rows 16b + 4*(lane/16) + e.  Only
  // the M real token rows go through LDS (one of sixteen at M = 1).
  float* red = reinterpret_cast<float*>(lds);  // [waves][16*NB tokens][kDecCols channels]
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (16 * b + 4 * g + e < M)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
          red[(wave * RR + 16 * b + 4 * g + e) * kDecCols + 16 * j + (lane & 15)] = acc[b][j][e];
  __syncthreads();
  // Each thread takes 4 adjacent channels (16 bytes of fp32) of token rows
  // tid/QPR + RPP*p, p = 0 .. NP-1.
  constexpr int QPR = kDecCols / 4;          // 4-channel groups per row
  constexpr int RPP = kDecThreads / QPR;     // token rows per pass
  constexpr int NP = (RR + RPP - 1) / RPP;   // passes covering 16*NB rows
  const int q = tid % QPR, c4 = n0 + 4 * q, mt = tid / QPR;
  const bool inb = c4 < H;  // H is a multiple of 8, so all 4 channels are in range
  const uint32_t mbits = inb && mask != nullptr ? *reinterpret_cast<const uint32_t*>(mask + c4) : 0u;
  bool syn[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) syn[e] = ((mbits >> (8 * e)) & 0xffu) != 0;
  f32x4_t y[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int m = mt + RPP * p;
    if (m < M) {
      y[p] = *reinterpret_cast<const f32x4_t*>(red + (0 * RR + m) * kDecCols + 4 * q);
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) y[p] += *reinterpret_cast<const f32x4_t*>(red + (w * RR + m) * kDecCols + 4 * q);
    }
  }
  // bf16 output of 4 channels of token row m of rank u: one 8-byte store.
  auto put = [&](int u, int m, f32x4_t v) {
    u32x2 pk;
    pk[0] = pack_bf16x2(v[0], v[1]);
    pk[1] = pack_bf16x2(v[2], v[3]);
    *reinterpret_cast<u32x2*>(out + u * os + (long long)m * H + c4) = pk;
  };
  // A channel block without synced channels (the same for all T workgroups
  // of the block; every block when mask == nullptr) needs no exchange and
  // no workspace when the contraction is whole: each rank writes its own
  // values.
  if (ks == 1 && !__syncthreads_or(mbits != 0u)) {
    if (inb)
#pragma unroll
      for (int p = 0; p < NP; ++p)
        if (mt + RPP * p < M) put(t, mt + RPP * p, y[p]);
    return;
  }

  // Otherwise every workgroup publishes its fp32 values [M][128] of rank t
  // (device-scope coherent sc1 16-byte stores) and counts itself in; the
  // last of the T to arrive reads all T ranks' values, adds them in
  // ascending rank order on the synced channels and writes every rank's
  // output: the sum on synced channels, the rank's own value elsewhere.
  // Waiting for the stores' acknowledgement before the arrival is counted
  // orders them; the coherent accesses need no cache write-back or
  // invalidation across the chip's L2 slices.
  // This handoff rests on gfx950's cache-policy bits, not on the HIP memory
  // model: the partials go through the sc1 (device-coherent) store and load
  // forms, which bypass the non-coherent per-XCD L2 for those lines, and the
  // counter is a relaxed device-scope atomic ordered by s_waitcnt.  A release
  // / acquire pair writes back and invalidates the whole L2 of the XCD
  // instead: as a per-wave fence 4x slower; on the one arrival atomic per
  // workgroup (acq_rel, agent scope, plain partial accesses; same bits)
  // M = 1 / 8 / 32 took 21.5 / 23.1 / 28.2 us against 18.8 / 19.3 / 23.0.  The bitwise decode
  // tests (chunked calls, a shared workspace, graph replays) guard it.
  constexpr int kSc1 = 1 << 4;
  // Slice sl of rank u sits at partial + (sl * T + u) * M * H.
  auto prs = [&](int u) { return make_rsrc(partial + u * MH, (uint32_t)(MH * 4)); };
  if (inb) {
    const __amdgpu_buffer_rsrc_t r = prs(sl * T + t);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int m = mt + RPP * p;
      if (m < M) __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, y[p]), r, (m * H + c4) * 4, 0, kSc1);
    }
  }
  __shared__ int is_last;
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(arrivals + blk, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == T * ks - 1;
  __syncthreads();
  if (!is_last) return;
  if (tid == 0) __hip_atomic_store(arrivals + blk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (!inb) return;
  // Ranks are taken 8 at a time, all their loads (every pass) in flight
  // together; with T <= 8 the loaded values also give the local channels.
  auto sel = [&](f32x4_t a, f32x4_t b) {  // synced channels from a, the rest from b
    f32x4_t r;
#pragma unroll
    for (int e = 0; e < 4; ++e) r[e] = syn[e] ? a[e] : b[e];
    return r;
  };
  if (SL && ks > 1) {
    // T * ks <= 8: every slice of every rank in flight together; each rank's
    // value is its slices' sum in slice order.
    const int n = T * ks;
    f32x4_t v[NP][8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (k < n) {
        const __amdgpu_buffer_rsrc_t r = prs(k);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int m = mt + RPP * p;
          if (m < M) v[p][k] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (m * H + c4) * 4, 0, kSc1));
        }
      }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int m = mt + RPP * p;
      if (m >= M) continue;
      f32x4_t vr[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (u < T) {
          vr[u] = v[p][u];
#pragma unroll
          for (int k = u + 1; k < 8; ++k)  // k = q * T + u: slices q = 1 .. ks - 1, in order
            if (k < n && (k - u) % T == 0) vr[u] += v[p][k];
        }
      f32x4_t sum = vr[0];
#pragma unroll
      for (int u = 1; u < 8; ++u)
        if (u < T) sum += vr[u];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (u < T) put(u, m, sel(sum, vr[u]));
    }
    return;
  }
  for (int u0 = 0; u0 < T; u0 += 8) {
    f32x4_t v[NP][8];
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (u0 + k < T) {
        const __amdgpu_buffer_rsrc_t r = prs(u0 + k);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const int m = mt + RPP * p;
          if (m < M) v[p][k] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (m * H + c4) * 4, 0, kSc1));
        }
      }
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (u0 + k < T) y[p] = (u0 + k == 0) ? v[p][k] : y[p] + v[p][k];
    if (T <= 8) {
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const int m = mt + RPP * p;
        if (m < M)
#pragma unroll
          for (int k = 0; k < 8; ++k)
            if (k < T) put(k, m, sel(y[p], v[p][k]));
      }
      return;
    }
  }
  // More than 8 ranks: a second pass re-reads each rank's own values.
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int m = mt + RPP * p;
    if (m < M)
      for (int u = 0; u < T; ++u)
        put(u, m, sel(y[p], __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(prs(u), (m * H + c4) * 4, 0, kSc1))));
  }
}

}  // namespace caat
