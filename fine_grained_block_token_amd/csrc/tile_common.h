// tile_common.h -- device helpers shared by the GEMM kernel files of libfgfp8:
// vector types, the K-block width, the LDS tile swizzle, the direct-to-LDS copy
// instructions, the XCD-aware tile order and the bf16 output store.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace fgfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBK = 128;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

// Byte offset of 16-byte chunk `chunk` (0..7) of tile row `row`: the chunk index
// is XORed with a key of the row's low three bits.  A fragment read has lane l
// on row r + (l & 15) at logical chunk 2(l >> 4) (+1), or l >> 4 (+4) for the
// group-32 layout.  Measured with ds_read_b128 on MI355X: the key
// (row & 7) ^ ((row >> 1) & 1) serves both layouts at the rate of a contiguous
// read (~190 B/clk/CU), at any stage offset; the key (row >> 1) & 7 runs the
// 16x16x128 layout at ~120 B/clk/CU (2-way bank conflicts).
__device__ __forceinline__ int swz_key(int row) { return (row & 7) ^ ((row >> 1) & 1); }
__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ swz_key(row)) << 4); }

typedef const void __attribute__((address_space(1))) *gptr_t;
typedef void __attribute__((address_space(3))) *lptr_t;

// 64 lanes x 16 bytes global -> LDS: lane l reads base + off (base wave-uniform,
// held in SGPRs; off a 32-bit per-lane offset) and its 16 bytes land at
// dst + 16*l (dst is wave-uniform and goes to M0).  Issued as inline assembly so
// that the compiler's wait insertion does not treat every later LDS read as
// possibly aliasing the copy in flight; the kernel orders these copies with
// explicit s_waitcnt vmcnt + s_barrier.
__device__ __forceinline__ void load_lds16(const void *base, uint32_t off, uint8_t *dst_wave) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lptr_t)dst_wave;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

// As load_lds16 with 4 bytes per lane (lane l's dword lands at dst + 4*l).
__device__ __forceinline__ void load_lds4(const void *base, uint32_t off, uint8_t *dst_wave) {
  const uint32_t lds = (uint32_t)(uintptr_t)(lptr_t)dst_wave;
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               ::"v"(off), "s"(base), "s"(lds) : "memory", "m0");
}

// Round 4 fp32 values to bf16 (nearest, ties to even) and store them at dp (8-byte
// aligned), only the first `left` when fewer than 4 columns remain.
__device__ __forceinline__ void store_bf16x4(uint16_t *dp, const v4f &v, int64_t left) {
  if (left >= 4) {
    *reinterpret_cast<u32x2 *>(dp) =
        (u32x2){bf16_rne(v[0]) | (bf16_rne(v[1]) << 16), bf16_rne(v[2]) | (bf16_rne(v[3]) << 16)};
  } else {
    for (int r = 0; r < left; ++r) dp[r] = (uint16_t)bf16_rne(v[r]);
  }
}

// Tile of workgroup blockIdx.x: block b runs on XCD b % 8, each XCD takes a
// contiguous range of tile ids, walked in bands of kGroupM m-tiles, so that the
// tiles resident on one XCD share A and B panels in its L2.  False for the
// workgroups past the last tile (the grid is a whole number of XCD ranges).
template <class C>
__device__ __forceinline__ bool tile_origin(int tiles_m, int tiles_n, int64_t &m0, int64_t &n0) {
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const int tid = (int)(blockIdx.x % kXcds) * per_xcd + (int)(blockIdx.x / kXcds);
  if (tid >= tiles) return false;
  const int band = tid / (kGroupM * tiles_n);
  const int band_m = min(kGroupM, tiles_m - band * kGroupM);
  const int in_band = tid - band * kGroupM * tiles_n;
  m0 = (int64_t)(band * kGroupM + in_band % band_m) * C::kBM;
  n0 = (int64_t)(in_band / band_m) * C::kBN;
  return true;
}

}  // namespace fgfp8
