// stage.h — staging of operand tiles in LDS and the matrix-core helpers
// shared by the bf16 kernels.
//
// Tiles go from global memory straight into LDS through the load units
// (global_load_lds), one 1 KB block per wave instruction, and are read back
// as 32x32x16 MFMA fragments, either along their rows (ds_read_b128) or
// across them (ds_read_b64_tr_b16, which hands every lane one column of
// four rows).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device.h"

namespace bd {

typedef __attribute__((address_space(3))) const void lds_void;

// Copies 16 (4) bytes per lane from global memory at sbase + voff into LDS
// at `lds` + 16 lane (4 lane); sbase and lds are the same for the whole wave.
// Written as inline assembly so the compiler does not order the copy
// against unrelated LDS reads; completion is awaited explicitly
// (wait_copies) before the barrier that publishes the data.  M0 (the LDS
// address) needs one wait state before the copy reads it.
__device__ __forceinline__ void copy16(const void* sbase, uint32_t voff, const void* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)(lds_void*)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(la)
               : "memory", "m0");
}
__device__ __forceinline__ void copy4(const void* sbase, uint32_t voff, const void* lds) {
  const uint32_t la = (uint32_t)(uintptr_t)(lds_void*)lds;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(la)
               : "memory", "m0");
}
// Marks a value that is the same in every lane as such (scalar registers).
__device__ __forceinline__ int32_t uniform(int32_t x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int32_t)x);
  const int32_t hi = __builtin_amdgcn_readfirstlane((int32_t)(x >> 32));
  return ((int64_t)hi << 32) | lo;
}
__device__ __forceinline__ void wait_copies() { __builtin_amdgcn_s_waitcnt(0x0f70); }  // vmcnt(0)
// Barrier that orders this wave's LDS writes before its partners' reads,
// without waiting for the copies still in flight.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Barrier that publishes this wave's LDS writes while the N LDS reads it
// issued after them stay in flight: a wave's LDS operations complete in
// order, so lgkmcnt(N) covers every write issued before those reads.  The
// caller pins the order (no scalar memory operation may be outstanding,
// those complete out of order).
template <int N>
__device__ __forceinline__ void barrier_lds_behind() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt holds 0..15");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f | (N << 8));  // lgkmcnt(N)
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Barrier for a wave that publishes no LDS writes: its reads stay in flight.
__device__ __forceinline__ void barrier_reads_in_flight() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


// Staged tiles are unpadded; 16-byte chunk c of row r sits at chunk
// position c ^ swz(r).  The LDS serves 256 bytes per cycle: a 128-bit read
// 16 lanes at a time, a 64-bit read 32 lanes at a time.  A fragment read
// along the rows touches one chunk of 16 consecutive rows; a transposed
// read touches four chunks (64 bytes) of four consecutive rows, rows
// 4i .. 4i+3.  Both land on distinct bank groups when swz maps the low two
// row bits to the high chunk bits and bits 2-3 to the low chunk bits:
//   256-byte rows: swz(r) = ((r & 3) << 2) | ((r >> 2) & 3)
//   128-byte rows (two rows per 256-byte bank line, told apart by r & 1):
//                  swz(r) = (((r >> 1) & 1) << 2) | ((r >> 2) & 3)
template <int NC>  // chunks per row: 16 (256-byte rows) or 8 (128-byte rows)
__host__ __device__ constexpr int swz(int r) {
  static_assert(NC == 16 || NC == 8, "rows of 128 or 256 bytes");
  return NC == 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// Per-lane element offsets into the swizzled tiles.  A fragment read takes
// logical chunk 2 k + hh (k-th 16-element step, lane half hh) of row
// 32 m + ql; swz(32 m + ql) = swz(ql).
// Tiles stage 64 rows: natural tiles are [64][D] bf16 (D / 8 chunks per
// row), transposed tiles [D][64] fp16 (8 chunks per row).
constexpr int kTileRows = 64;

template <int D>
struct LaneOff {
  int nat[D / 16];          // natural rows (D / 8 chunks)
  int tr[kTileRows / 16];   // transposed rows (8 chunks)
  int ntr[2][D / 32];       // transposed reads of natural tiles: [half][32-column block]
  uint32_t dn[2];           // byte offsets of this lane's chunk in its even / odd copy blocks (natural)
  uint32_t dt;              // byte offset of this lane's chunk in every copy block (transposed)
};

// Offsets for a workgroup of NW waves whose wave w copies 1 KB blocks
// w, w + NW, ... of every tile (the j-th of them with dn[j & 1]).
template <int D, int NW>
__device__ inline LaneOff<D> lane_offsets(int wave, int lane) {
  constexpr int NCR = D / 8;  // chunks per natural row
  static_assert((2 * NW * 64 / NCR) % 16 == 0 && (NW * 8) % 16 == 0,
                "a wave's copy blocks two apart keep its rows' swizzle");
  const int ql = lane & 31, hh = lane >> 5;
  LaneOff<D> o;
#pragma unroll
  for (int k = 0; k < D / 16; ++k) o.nat[k] = ((2 * k + hh) ^ swz<NCR>(ql)) * 8;
#pragma unroll
  for (int k = 0; k < kTileRows / 16; ++k) o.tr[k] = ((2 * k + hh) ^ swz<8>(ql)) * 8;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int p = (wave + NW * j) * 64 + lane;  // physical chunk in the wave's j-th 1 KB block
    const int row = p / NCR;
    o.dn[j] = (uint32_t)(row * D + ((p % NCR) ^ swz<NCR>(row)) * 8 - (NW * j * 64 / NCR) * D) * 2;
  }
  const int p = wave * 64 + lane;  // physical chunk of the wave's first 1 KB block
  const int d = p / 8;
  o.dt = (uint32_t)(d * kTileRows + ((p % 8) ^ swz<8>(d)) * 8) * 2;
  // Transposed read of a natural tile (see tr_frag): lane 16 G + 4 j + q
  // points at row 8 h + 4 (G / 2) + j, columns 32 db + 16 (G % 2) + 4 q .. +4
  // (rows of a 16-row step relative to its first row).
  const int G = lane >> 4, j = (lane >> 2) & 3, q = lane & 3;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int row = 8 * h + 4 * (G >> 1) + j, col = 32 * db + 16 * (G & 1) + 4 * q;
      o.ntr[h][db] = row * D + (((col >> 3) ^ swz<NCR>(row)) << 3) + (col & 7);
    }
  return o;
}

// MFMA A operand T^T[m = column][k = row] of rows 16 s .. 16 s + 15 and
// columns 32 db .. 32 db + 31 of a natural fp16 tile T (D columns), read
// across the rows.  Within each group of 16 lanes the transposed read
// gives lane i, element e, the (i % 4)-th value at the address of lane
// 4 e + i / 4; with the addresses of lane_offsets, lane l receives column
// 32 db + l % 32 of rows 16 s + 8 h + 4 (l / 32) + e, e = 0..3, for the two
// halves h.  That is the row order in which an MFMA C tile hands its rows
// over as a B operand (device.h), so no row permutation is stored.
typedef __attribute__((__vector_size__(4 * sizeof(__fp16)))) __fp16 fp16x4_tr;
typedef __attribute__((address_space(3))) fp16x4_tr lds_fp16x4_tr;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
template <int D>
__device__ __forceinline__ f16x8 tr_frag(const _Float16* step, const LaneOff<D>& o, int db) {
  const fp16x4_tr lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_tr*)(lds_void*)(step + o.ntr[0][db]));
  const fp16x4_tr hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_fp16x4_tr*)(lds_void*)(step + o.ntr[1][db]));
  return __builtin_shufflevector(__builtin_bit_cast(f16x4, lo), __builtin_bit_cast(f16x4, hi), 0, 1, 2, 3, 4, 5,
                                 6, 7);
}

// Fragment reads kept in flight ahead of the products that consume them;
// scheduling barriers pin this order (the compiler otherwise sinks each
// read to its first use).  Measured at 2..10 on the 64K workload: 2-4 are
// best (about 2% over 6); deeper queues only lengthen the LDS queue.
constexpr int kAhead = 4;

// C^T blocks of one staged natural tile: acc[kb] = tile[kb*32 .. +32][:]
// times the lane's row held in registers (B operand), for the two 32-row
// blocks of a 64-row tile; fragment f = (ks, kb), kAhead reads in flight.
template <int D>
__device__ __forceinline__ void scores_2kb(const uint16_t* tile, int ql, const bf16x8 (&row)[D / 16],
                                           const LaneOff<D>& o, f32x16 (&acc)[2]) {
  constexpr int NF = 2 * (D / 16);
  const uint16_t* tb = tile + ql * D;
  bf16x8 fr[NF];
#pragma unroll
  for (int f = 0; f < kAhead; ++f) fr[f] = ld16<bf16x8>(tb + (f & 1) * 32 * D + o.nat[f >> 1]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + kAhead < NF) {
      const int h = f + kAhead;
      fr[h] = ld16<bf16x8>(tb + (h & 1) * 32 * D + o.nat[h >> 1]);
    }
    const int kb = f & 1, ks = f >> 1;
    acc[kb] = mfma_bf16(fr[f], row[ks], ks ? acc[kb] : f32x16{});
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Two C^T blocks of 32 rows of staged natural fp16 tiles (starting at
// block_a, block_b) times the lane's fp16 rows held in registers, their
// products interleaved: acc_a = block_a row_a^T, acc_b = block_b row_b^T.
// Two independent accumulation chains
// let each product issue while the other chain's last result is still in
// flight (measured on the dQ kernel: -1.6% against one chain after the
// other); two reads per chain stay in flight ahead of the products.
template <int D>
__device__ __forceinline__ void scores_1kb_pair_f16(const _Float16* block_a, const f16x8 (&row_a)[D / 16],
                                                    const _Float16* block_b, const f16x8 (&row_b)[D / 16], int ql,
                                                    const LaneOff<D>& o, f32x16& acc_a, f32x16& acc_b) {
  constexpr int NF = D / 16, AH = 2;
  const _Float16* ta = block_a + ql * D;
  const _Float16* tb = block_b + ql * D;
  f16x8 fa[NF], fb[NF];
#pragma unroll
  for (int f = 0; f < AH; ++f) {
    fa[f] = ld16<f16x8>(ta + o.nat[f]);
    fb[f] = ld16<f16x8>(tb + o.nat[f]);
  }
  __builtin_amdgcn_sched_barrier(0);
  acc_a = f32x16{};
  acc_b = f32x16{};
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if (f + AH < NF) {
      fa[f + AH] = ld16<f16x8>(ta + o.nat[f + AH]);
      fb[f + AH] = ld16<f16x8>(tb + o.nat[f + AH]);
    }
    acc_a = mfma_f16(fa[f], row_a[f], acc_a);
    acc_b = mfma_f16(fb[f], row_b[f], acc_b);
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace bd
