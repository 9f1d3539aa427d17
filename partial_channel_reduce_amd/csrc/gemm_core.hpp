// bf16 MFMA GEMM building blocks for gfx950 (CDNA4).
//
// A workgroup of NW wave64s (a 2 x NW/2 grid) owns a BM x BN output tile and
// walks the contraction in 64-wide chunks, double buffered in LDS.  Each wave
// accumulates its (BM/2) x (2*BN/NW) sub-tile with v_mfma_f32_32x32x16_bf16
// (fp32 accumulation).  With NW = 8 two waves share each SIMD, so one wave's
// LDS and barrier waits are covered by the other's MFMAs.
//
// Operands are described by where their contraction index k is contiguous in
// global memory, and each kind keeps that orientation in LDS:
//   * KCONT  [row][k]: LDS tile [R rows][64 k], 128 B rows, 16-byte chunks XOR
//            swizzled by row; an MFMA fragment (8 consecutive k of one row) is
//            one ds_read_b128.
//   * MNCONT [k][row]: LDS tile [64 k][R rows], 2R-byte rows, 16-byte chunks
//            XOR swizzled by k; a fragment is gathered and transposed by two
//            ds_read_b64_tr_b16 (gfx950's LDS transpose read: within each
//            16-lane group, lane 4s+u names 4 consecutive rows of k-row s, and
//            every lane receives one row's values from the 4 k-rows).
// Every operand is copied global -> LDS with buffer_load_dwordx4 ... lds (no
// register staging).
#pragma once

#include "common.hpp"

namespace caat {

constexpr int kBK = 64;

typedef __attribute__((address_space(3))) void lds_void_t;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;

template <int BM, int BN, int NW = 4>
struct TileShape {
  static constexpr int THREADS = NW * 64;
  static constexpr int WGM = 2, WGN = NW / 2;       // waves along BM, BN
  static constexpr int WM = BM / WGM, WN = BN / WGN;  // per-wave sub-tile
  static constexpr int WI = WM / 32, WJ = WN / 32;  // 32x32 MFMA blocks per wave
  static constexpr int BUF = (BM + BN) * kBK;       // one stage, bf16 elements
  static constexpr int LDS_ELEMS = 2 * BUF;         // double buffer
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(BM % 64 == 0 && BN % 64 == 0 && WM % 32 == 0 && WN % 32 == 0, "tile must be a multiple of 64");
};

// Accumulators of one wave: WI x WJ blocks of 32x32 fp32.
template <int BM, int BN, int NW>
using AccTile = f32x16[TileShape<BM, BN, NW>::WI][TileShape<BM, BN, NW>::WJ];

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---- LDS layouts ----------------------------------------------------------------
// The LDS serves 256 bytes (64 banks) per cycle, i.e. 16 lanes of a 16-byte
// read or 32 lanes of an 8-byte read at a time; the swizzles below keep each
// such group on distinct banks.
//
// KCONT: element offset of 16-byte chunk `chunk` (0..7) of row `row`.  Rows are
// 128 bytes, so a 16-row group spans two rows per bank set; XOR with
// (row / 2) % 8 gives its 16 rows 16 distinct (row parity, chunk) slots.
__device__ __forceinline__ int kc_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int kc_off(int row, int chunk) { return row * kBK + ((chunk ^ kc_swz(row)) << 3); }
// MNCONT with R elements per k-row: element offset of logical chunk `chunk`
// (0..R/8-1) of k-row `k`.  A transpose read by 32 lanes covers 4 k-rows x 4
// consecutive chunks; XOR with 4 * (k % 4) puts them on 16 distinct chunks.
template <int R>
__device__ __forceinline__ int mn_off(int k, int chunk) { return k * R + ((chunk ^ ((k & 3) << 2)) << 3); }

// ---- direct global -> LDS copies (one wave instruction moves 1 KiB) -------------
// Buffer loads with an LDS destination.  The per-lane part of the address is
// the same for every instruction of a tile (one VGPR), the rest is a uniform
// SGPR offset; reads past the end of the buffer return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)nbytes, 0x00020000);
}

// Workgroup barrier for LDS hand-offs: each wave first completes its own LDS
// accesses; the caller has already waited for whatever copies into LDS the
// other waves need.  Unlike __syncthreads() it carries no fence, which would
// also wait for every outstanding global access of the wave (prefetches,
// stores) although nothing after the barrier depends on them.  The memory
// clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One wave-wide 16-byte-per-lane copy global -> LDS: lane i's 16 bytes from
// rsrc + voff + soff land at lds + 16 * i.  Written as inline assembly on
// purpose: the compiler cannot tell which LDS bytes such a copy writes, and
// if it sees the copy it makes every later LDS read wait until the copy has
// finished -- which would stall the reads of the current stage behind the
// loads of the next one.  Users order these copies explicitly: a wait for
// all of the wave's memory operations, then a workgroup barrier, before the
// destination is read, and no copy into a buffer that is still being read.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, const void* lds, int voff, int soff) {
  const uint32_t la = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" : : "s"(la), "v"(voff), "s"(rsrc),
               "s"(soff));
}

// KCONT tile: rows r0..r0+R-1 of a row-major [rows][ld] buffer, k0..k0+63.
// Rows past the buffer read as zero; k past the contraction reads the next
// row's values, which the caller clears (zero_kcont_tail).
struct KcDma {
  __amdgpu_buffer_rsrc_t rsrc;
  int voff;  // bytes: this lane's (row in group of 8, swizzled chunk)
  // The wave's instructions cover 8-row groups whose index has the wave's
  // parity, so kc_swz(row) is the same for all of them.
  __device__ __forceinline__ KcDma(const void* base, uint32_t nbytes, int ld, int lane, int wave) {
    rsrc = make_rsrc(base, nbytes);
    const int r = lane >> 3;
    voff = (r * ld + (((lane & 7) ^ kc_swz((wave & 1) * 8 + r)) << 3)) * 2;
  }
  template <int R, int NW>
  __device__ __forceinline__ void load(int ld, int r0, int k0, uint16_t* tile, int wave) const {
#pragma unroll
    for (int i = 0; i < R / (8 * NW); ++i) {
      const int rb = (i * NW + wave) * 8;  // 8 rows per instruction
      // byte offsets in unsigned 32-bit arithmetic: rows past the end of the
      // buffer may take them past 2^31, where they read as zero
      const int soff = __builtin_amdgcn_readfirstlane((int)(((uint32_t)(r0 + rb) * (uint32_t)ld + (uint32_t)k0) * 2u));
      dma16(rsrc, tile + rb * kBK, voff, soff);
    }
  }
};

// MNCONT tile: k-rows k0..k0+63 of a row-major [k][ld] buffer, columns
// c0..c0+R-1.  k-rows past the buffer read as zero.
template <int R>
struct MnDma {
  static constexpr int CPR = R / 8;     // 16-byte chunks per k-row
  static constexpr int RPI = 64 / CPR;  // k-rows per instruction
  __amdgpu_buffer_rsrc_t rsrc;
  int voff;
  __device__ __forceinline__ MnDma(const void* base, uint32_t nbytes, int ld, int lane, int wave) {
    rsrc = make_rsrc(base, nbytes);
    const int kr = lane / CPR;                 // k-row within the instruction
    const int k = (wave * RPI + kr) & 3;       // (row in tile) % 4, the same for every instruction
    const int chunk = (lane % CPR) ^ (k << 2);  // logical chunk stored at this lane's slot
    voff = (kr * ld + chunk * 8) * 2;
  }
  template <int NW>
  __device__ __forceinline__ void load(int ld, int c0, int k0, uint16_t* tile, int wave) const {
#pragma unroll
    for (int i = 0; i < R / (8 * NW); ++i) {
      const int kb = (i * NW + wave) * RPI;
      const int soff = __builtin_amdgcn_readfirstlane((int)(((uint32_t)(k0 + kb) * (uint32_t)ld + (uint32_t)c0) * 2u));
      dma16(rsrc, tile + kb * R, voff, soff);
    }
  }
};

// Zero the part of a staged KCONT chunk that lies beyond the contraction
// (k >= kvalid within the chunk).  Called after the chunk has landed and
// before it is read.
template <int R, int NTHREADS>
__device__ __forceinline__ void zero_kcont_tail(uint16_t* tile, int kvalid, int tid) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  const int c0 = kvalid >> 3;  // first 16-byte chunk to clear (kvalid % 8 == 0)
  for (int q = tid; q < R * 8; q += NTHREADS) {
    const int row = q >> 3, c = q & 7;
    if (c >= c0) st16(tile + kc_off(row, c), z);
  }
}

// ---- fragments ------------------------------------------------------------------
// KCONT fragment of 32 rows starting at rb, k16 step ks: lane l gets row rb+l%32,
// k = ks*16 + 8*(l/32) .. +7.
__device__ __forceinline__ u32x4 frag_kcont(const uint16_t* tile, int rb, int ks, int lane) {
  return ld16(tile + kc_off(rb + (lane & 31), ks * 2 + (lane >> 5)));
}
// MNCONT fragment of 32 rows starting at rb: same lane layout as frag_kcont,
// gathered from the [k][R] tile by two transpose reads.
template <int R>
__device__ __forceinline__ u32x4 frag_mncont(const uint16_t* tile, int rb, int ks, int lane) {
  const int g = lane >> 4, jj = lane & 15, s = jj >> 2, u = jj & 3;
  const int col = rb + 16 * (g & 1) + 4 * u;  // first of the 4 rows this lane names
  const int kbase = ks * 16 + 8 * (g >> 1) + s;
  u32x4 r;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int k = kbase + 4 * h;
    const int off = mn_off<R>(k, col >> 3) + (col & 7);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + off));
    const u32x2 w = __builtin_bit_cast(u32x2, v);
    r[2 * h] = w[0];
    r[2 * h + 1] = w[1];
  }
  return r;
}

// Row (within a 32x32 block) of accumulator register e of `lane`; the column is lane % 32.
__device__ __forceinline__ int acc_row(int e, int lane) { return (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3); }

// Grouped raster of a tiles_m x tiles_n grid: GROUP m-tiles are walked column
// by column, so tiles running together share B columns and nearby A rows.
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

template <int BM, int BN, int NW>
__device__ __forceinline__ void zero_acc(AccTile<BM, BN, NW>& acc) {
#pragma unroll
  for (int i = 0; i < TileShape<BM, BN, NW>::WI; ++i)
#pragma unroll
    for (int j = 0; j < TileShape<BM, BN, NW>::WJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
}

// One 64-wide chunk of MFMAs.  Fragments for k16 step ks+1 are read while the
// MFMAs of step ks run, and `pre` (the next chunk's global loads) is issued
// during step 0: the schedule alternates one MFMA with one LDS read and one
// global load, so neither the LDS nor the load queue issues in a burst that
// would leave the matrix core idle.
// fa(ks, i) / fb(ks, j) return the A / B fragments of block i / j.
template <int BM, int BN, int NW, class FA, class FB, class PRE>
__device__ __forceinline__ void mma_chunk(FA&& fa, FB&& fb, AccTile<BM, BN, NW>& acc, PRE&& pre) {
  using S = TileShape<BM, BN, NW>;
  constexpr int NM = S::WI * S::WJ;
  u32x4 a[2][S::WI], b[2][S::WJ];
  // Fragments are read in the order the MFMAs (i-major) consume them: A0 and
  // every B first, then the remaining A, so each has most of a k-step to land.
  auto read = [&](int ks, int p) {
    a[p][0] = fa(ks, 0);
#pragma unroll
    for (int j = 0; j < S::WJ; ++j) b[p][j] = fb(ks, j);
#pragma unroll
    for (int i = 1; i < S::WI; ++i) a[p][i] = fa(ks, i);
  };
  read(0, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < kBK / 16; ++ks) {
    if (ks == 0) pre();
    if (ks + 1 < kBK / 16) read(ks + 1, (ks + 1) & 1);
#pragma unroll
    for (int i = 0; i < S::WI; ++i)
#pragma unroll
      for (int j = 0; j < S::WJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[ks & 1][i]), as_bf16x8(b[ks & 1][j]),
                                                            acc[i][j], 0, 0, 0);
#pragma unroll
    for (int x = 0; x < NM; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one global load
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ---- epilogue staging -----------------------------------------------------------
// A wave's accumulators hold the transpose of its output sub-tile: MFMA rows
// are the output's contiguous index, MFMA columns its row index, so a lane
// owns 4 consecutive outputs of one row per register group.  Written straight
// to memory that would make every store instruction touch 64 rows.  Instead
// the sub-tile is staged in LDS as [row][WC] bf16 (16-byte chunks XOR
// swizzled by row) and read back in row order, so each store instruction
// writes whole 128-byte lines.
template <int WC>  // contiguous extent of the sub-tile (elements, multiple of 64)
struct RowStage {
  static constexpr int CPR = WC / 8;    // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;  // rows per wave instruction
  static __device__ __forceinline__ int off(int r, int c) { return r * WC + ((c ^ (r & (CPR - 1))) << 3); }
  // Block (i, *) of the accumulators into rows row0 .. row0+31.
  static __device__ __forceinline__ void put(uint16_t* st, const f32x16& a, int i, int row0, int lane) {
    const int r = row0 + (lane & 31);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = i * 4 + q;
      u32x2 v;
      v[0] = pack_bf16x2(a[4 * q], a[4 * q + 1]);
      v[1] = pack_bf16x2(a[4 * q + 2], a[4 * q + 3]);
      *reinterpret_cast<u32x2*>(st + off(r, c) + (lane >> 5) * 4) = v;
    }
  }
  // The same from bf16 already packed in pairs: word w holds the values of
  // accumulator registers 2w and 2w+1.
  static __device__ __forceinline__ void put_packed(uint16_t* st, const uint32_t (&p)[8], int i, int row0, int lane) {
    const int r = row0 + (lane & 31);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x2 v = {p[2 * q], p[2 * q + 1]};
      *reinterpret_cast<u32x2*>(st + off(r, i * 4 + q) + (lane >> 5) * 4) = v;
    }
  }
  // Rows 0 .. nrows-1 in row order: store(r, c, v) gets chunk c of row r.
  template <class F>
  static __device__ __forceinline__ void drain(const uint16_t* st, int nrows, int lane, F&& store) {
    const int rl = lane / CPR, c = lane % CPR;
#pragma unroll 4
    for (int r0 = 0; r0 < nrows; r0 += RPI) {
      const int r = r0 + rl;
      store(r, c, ld16(st + off(r, c)));
    }
  }
};

}  // namespace caat
