// Tile staging shared by the bf16 MFMA attention kernels (gfx950).
//
// Tiles go from global memory straight into LDS with global_load_lds_dwordx4:
// each lane of a wavefront fetches 16 bytes from an address of its own and the
// hardware writes them at (LDS base) + 16 * lane, so one instruction fills one
// contiguous 1 KB block and no registers hold the data in flight.  Since the
// blocks are contiguous, LDS rows cannot be padded; bank conflicts are avoided
// instead by XOR-swizzling the 16-byte chunks of each row: logical chunk c of
// row r is stored at chunk c ^ swz(r).  The LDS has 64 four-byte banks (16
// groups of 16 bytes).  Two read patterns must be conflict-free:
//  - MFMA operand reads (ds_read_b128, 16 lanes per cycle): 16 consecutive
//    rows at the same logical chunk, so swz must take 16 different values
//    over any 16 consecutive rows (per bank-alignment class of the rows);
//  - transposing reads (ds_read_b64_tr_b16, 32 lanes per cycle): 4 consecutive
//    rows x 4 consecutive chunks (64 bytes), so the 4 rows must land in 4
//    different 4-chunk groups.
// For 256-byte rows swz(r) = ((r & 3) << 2) | ((r >> 2) & 3); for 128-byte rows
// (two rows per 16 bank groups) the same idea on x = (r >> 1) & 7.
//
// MFMA operand reads (v_mfma_f32_32x32x16_bf16): lane (ln, hf) = (lane % 32,
// lane / 32) reads row ln of a 32-row block, logical chunk 2c + hf, i.e. the 8
// consecutive contraction elements 16c + 8hf .. +7 -- for row-major tiles
// (contraction over d) directly.  Operands contracted over keys or queries,
// whose B operand is a probability block in registers, need the contraction
// elements in the order {16c + 4hf + 0..3, 16c + 8 + 4hf + 0..3} (forced by the
// 32x32 result layout): transposed copies in global memory are stored by their
// producers with bits 2 and 3 of the column index swapped (see perm16), which
// makes that one 16-byte read; a row-major tile gives the same operand with
// two transposing reads (tr_frag).
#pragma once

#include "lh_internal.h"

namespace lh {
namespace tiles {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// column position of element m in a transposed copy: bits 2 and 3 swapped
__host__ __device__ __forceinline__ int perm16(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// chunk swizzle for rows of W bytes (W = 64, 128 or 256)
template <int W>
__host__ __device__ __forceinline__ int swz(int r) {
  static_assert(W == 64 || W == 128 || W == 256, "row width");
  if constexpr (W == 256) return ((r & 3) << 2) | ((r >> 2) & 3);
  if constexpr (W == 128) {
    const int x = (r >> 1) & 7;
    return ((x & 1) << 2) | (x >> 1);
  }
  return (r >> 2) & 3;
}

// byte offset of (row r, logical 16-byte chunk c) in a tile of W-byte rows
template <int W>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * W + 16 * (c ^ swz<W>(r));
}

__device__ __forceinline__ bf16x8 lds_frag(const char *tile, int off) {
  return *reinterpret_cast<const bf16x8 *>(tile + off);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element i % 4 of the 8-byte pieces addressed by lanes
// 4k + i / 4, k = 0..3.  So if lanes 4k .. 4k+3 of a group address the 16
// consecutive elements [c0, c0 + 16) of row r0 + k, lane i receives column
// c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ s16x4 lds_tr4(const char *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
}

// Per-lane byte offset, in a row-major tile of W-byte bf16 rows, of the
// transposing read that gives lane (ln, hf) column c0 + ln of rows
// r0 + 4 hf + 0..3 (lanes 4k + m of each 16-lane group address row r0 + 4 hf + k,
// columns c0 + 16 (group & 1) + 4m .. +3).
template <int W>
__device__ __forceinline__ int tr_off(int r0, int c0) {
  const int l = threadIdx.x & 63, li = l & 15;
  const int r = r0 + 4 * (l >> 5) + (li >> 2);
  const int col = c0 + 16 * ((l >> 4) & 1) + 4 * (li & 3);
  return r * W + 16 * ((col >> 3) ^ swz<W>(r)) + 2 * (col & 7);
}

// MFMA A operand of X^T for a row-major tile X (rows = contraction index):
// lane (ln, hf) gets column c0 + ln of rows {r0 + 4hf + 0..3, r0 + 8 + 4hf + 0..3}
// -- the probability-register order above -- from two transposing reads at the
// per-lane offsets lo = tr_off(r0, c0), hi = tr_off(r0 + 8, c0).
__device__ __forceinline__ bf16x8 tr_frag(const char *tile, int lo, int hi) {
  const s16x8 v = __builtin_shufflevector(lds_tr4(tile + lo), lds_tr4(tile + hi), 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// 32-bit LDS address of a pointer into __shared__ memory, the same in every lane
__device__ __forceinline__ unsigned lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(const __attribute__((address_space(3))) void *)p);
}

// One global->LDS load: lane l writes LDS bytes [lds + BYTES l, lds + BYTES (l+1))
// from gsrc (BYTES = 16 or 4).  The instruction is issued from asm rather than
// through the compiler's builtin: the compiler cannot tell which LDS buffer such
// a load writes, so after the builtin it makes the next LDS read of any buffer
// wait for the load to land -- which would serialize each tile's prefetch with
// the computation on the tile before it.  Ordering is the kernels' own: a
// wavefront waits for its loads (s_waitcnt vmcnt) and then meets the others at
// a barrier before any of them reads the tile.  M0 carries the LDS address; every
// other use of M0 in these kernels sets it right before use.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <int BYTES>
__device__ __forceinline__ void lds_load(const void *gsrc, unsigned lds) {
  static_assert(BYTES == 16 || BYTES == 4, "dwordx4 or dword");
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds), "v"(gsrc) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off" ::"s"(lds), "v"(gsrc) : "memory", "m0");
}
// The same with a scalar base address and a per-lane 32-bit offset: the base
// (the same in every lane) stays in scalar registers, so a kernel that keeps
// the per-lane offsets of its fills in registers spends no vector instructions
// on fill addresses.
template <int BYTES>
__device__ __forceinline__ void lds_load_s(const void *sbase, unsigned voff, unsigned lds) {
  static_assert(BYTES == 16 || BYTES == 4, "dwordx4 or dword");
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2" ::"s"(lds), "v"(voff), "s"(sbase)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Per-lane source offset, for lds_load_s, of 1 KB block b of a tile of W-byte
// rows whose rows lie gstride bytes apart in global memory (same swizzle as dma_tile).
template <int W>
__device__ __forceinline__ unsigned dma_voff(int b, unsigned gstride) {
  const int byte = b * 1024 + 16 * (int)(threadIdx.x & 63);
  const int r = byte / W;
  const int lc = ((byte % W) / 16) ^ swz<W>(r);
  return (unsigned)r * gstride + 16u * (unsigned)lc;
}

// Fill an R x W-byte tile: row r comes from gsrc + min(r, rclamp) * gstride.
// Every wavefront of the NT-thread work-group issues the same number of 1 KB
// blocks (a fixed trip count, so the fill adds no branches to the caller).
template <int W, int R, int NT>
__device__ __forceinline__ void dma_tile(char *lds_tile, const char *gsrc, long long gstride, int rclamp) {
  constexpr int BLOCKS = R * W / 1024, WAVES = NT / 64;
  static_assert(R * W % 1024 == 0 && BLOCKS % WAVES == 0, "whole 1 KB blocks, as many per wavefront");
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < BLOCKS / WAVES; ++i) {
    const int b = w + i * WAVES;
    const int byte = b * 1024 + 16 * l;
    const int r = byte / W;
    const int pc = (byte % W) / 16;
    const int lc = pc ^ swz<W>(r);
    lds_load<16>(gsrc + (long long)min(r, rclamp) * gstride + 16 * lc, lds_addr(lds_tile + b * 1024));
  }
}

// One dword per lane: lane l of the wavefront writes lds + 4 l from src.
__device__ __forceinline__ void dma_dword(void *lds, const void *src) { lds_load<4>(src, lds_addr(lds)); }

// wait for this wavefront's outstanding loads (the LDS fills included); a
// waitcnt written in the source is kept as written by the compiler
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0); }

// Wait until at most N of this wavefront's global loads are outstanding --
// loads complete in issue order, so every fill issued before the last N loads
// has landed -- and all its LDS reads have returned, then meet the other
// wavefronts of the work-group at a barrier.  One asm statement, so the
// compiler moves no memory access across it and adds no wait of its own (the
// fence of __syncthreads would wait for every outstanding load).  Used with
// fills issued two or more tiles ahead: N = the loads of the fills still
// allowed in flight.
template <int N>
__device__ __forceinline__ void wait_fills_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// The same, but leaving this wavefront's last M LDS reads in flight (LDS reads
// complete in issue order): for reads already issued from a tile that the
// fills after the barrier do not overwrite.
template <int N, int M>
__device__ __forceinline__ void wait_fills_barrier_keep() {
  static_assert(N >= 0 && N < 64 && M >= 0 && M < 16, "vmcnt / lgkmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(%1)\n\ts_barrier" ::"n"(N), "n"(M) : "memory");
}

}  // namespace tiles
}  // namespace lh
