// gemm_wide.hip -- 256x256-tile FP8 NT GEMM for power-of-two scales on gfx950.
//
// D = (A * 2^ea)(B * 2^eb)^T rounded to bf16: A [m, k] and B [n, k] E4M3, one
// exponent per row of A and 128-wide K block, one per 128x128 block of B (the
// GEMM of "DeepGEMM Essentials", Parts 1 and 6, with the UE8M0 scales of the
// per-token and per-block casts' UE8M0 option in "deep-gemm: fused per-token FP8
// cast in Triton").  The exponents are applied by V_MFMA_SCALE_F32_32X32X64_F8F6F4,
// which accumulates across all of K in fp32, so there is no per-block promotion
// and the accumulators need no second copy.
//
// Design (measured on MI355X):
//  * One workgroup of 4 waves per CU; each wave owns a 128x128 block of the
//    256x256 tile as 4x4 tiles of 32x32, 256 fp32 accumulators held in the
//    accumulation registers.  Per 128-wide K block a CU copies 64 KB for
//    256x256 outputs, half the bytes per flop of two 128x128 workgroups; one wave
//    per SIMD costs 12% of the MFMA issue rate (4.18 against 4.77 PF for
//    32x32x64 in a probe), less than the copies save.
//  * Two LDS stages of 66 KB (A 32 KB, B 32 KB, scales); the tile swizzle and
//    direct-to-LDS copies of gemm.hip.
//  * With one wave per SIMD no other wave covers a stall, so the next block's 16
//    tile copies per wave are spread one per MFMA over the first half of the
//    block's 32 MFMAs, and the other K half's fragments are read under the first
//    half's MFMAs.  The loop body is one basic block: the last step copies its own
//    block again (into the free stage) instead of branching, since a branch splits
//    the block and the compiler then sinks all MFMAs below all copies (measured:
//    that schedule ran 5% slower than the 128x128 kernel, this one 5-10% faster).
//  * Results are bit-identical to gemm_g32_kernel's (measured on every test shape).
// This file is compiled without --amdgpu-mfma-vgpr-form, so that the MFMAs keep
// their accumulators in the accumulation registers.
#include "gemm_wide.h"

#include "device_common.h"
#include "tile_common.h"

namespace fgfp8 {
namespace {

typedef float v16f __attribute__((ext_vector_type(16)));

struct WideCfg {
  static constexpr int kBM = 256, kBN = 256, kWaves = 4, kThreads = 256;
  static constexpr int kABytes = kBM * kBK, kBBytes = kBN * kBK;
  static constexpr int kSaOff = kABytes + kBBytes;   // 256 row exponents (fp32 2^e or packed words)
  static constexpr int kSbOff = kSaOff + 4 * kBM;    // 4 slots of 64 copies of a B block scale
  static constexpr int kStageBytes = 66 * 1024;      // a multiple of 512: the swizzle's bank pattern holds
  static constexpr int kALoads = kABytes / 1024 / kWaves, kBLoads = kBBytes / 1024 / kWaves;
  static_assert(kSbOff + 4 * 256 <= kStageBytes, "stage layout");
};

// MFMA operand of the 32x32x64 instruction: lane (r32 = l & 31, h = l >> 5) holds row
// r32 and K bytes [64h + 32s, 64h + 32s + 32) of the 128-wide block for the block's
// s-th MFMA (s = 0, 1).  A and B use the same K mapping.
__device__ __forceinline__ v8i frag32(const uint8_t *tile, int row, int h, int s) {
  const u32x4 lo = *reinterpret_cast<const u32x4 *>(tile + swz(row, 4 * h + 2 * s));
  const u32x4 hi = *reinterpret_cast<const u32x4 *>(tile + swz(row, 4 * h + 2 * s + 1));
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// Group-32 operand layout.  Measured on MI355X with one-hot K positions: the scale of
// lane r (r < 32) applies to bytes 0-15 (v0-3) of row r in both lane groups, the scale
// of lane r + 32 to bytes 16-31 (v4-7).  So lane (r32, h) of the block's MFMA s loads
// 16-byte chunk 4s + h of its row into v0-3 and chunk 4s + 2 + h into v4-7: the two
// v0-3 halves of a row form 32-K group 2s, the two v4-7 halves group 2s + 1, and lane
// (r32, h) carries the exponent of group 2s + h.  A and B use the same K order.
__device__ __forceinline__ v8i frag32_g32(const uint8_t *tile, int row, int h, int s) {
  const u32x4 lo = *reinterpret_cast<const u32x4 *>(tile + swz(row, 4 * s + h));
  const u32x4 hi = *reinterpret_cast<const u32x4 *>(tile + swz(row, 4 * s + 2 + h));
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// Exponent layouts: 1x128 A exponents as fp32 2^e or packed words (byte kb % 4 of
// word kb / 4) with one fp32 2^e per 128x128 block of B; or group 32 on both
// operands (one word per row or column and 128-K block, byte g for 32-K group g).
enum : int { kWideUeFloat = 0, kWideUePacked = 1, kWideG32 = 2 };

template <int MODE>
__global__ __launch_bounds__(WideCfg::kThreads, 1) void gemm_wide_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  constexpr bool G32 = MODE == kWideG32;
  using C = WideCfg;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::kStageBytes];
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = (wv >> 1) * 128, wn = (wv & 1) * 128;
  int64_t m0, n0;
  if (!tile_origin<C>(tiles_m, tiles_n, m0, n0)) return;
  const int64_t m = g.m, n = g.n;
  const int KB = (int)(g.k / kBK);
  const int64_t nbl = (n + 127) / 128;

  // copy c < kALoads: A rows 8(4c + wv) .. +7; else B rows likewise (rows past the
  // matrix edge read its last row; their results are never stored)
  uint32_t off[C::kALoads + C::kBLoads];
#pragma unroll
  for (int i = 0; i < C::kALoads; ++i) {
    const int sl = 64 * (i * C::kWaves + wv) + lane, row = sl >> 3, chunk = (sl & 7) ^ swz_key(row);
    off[i] = (uint32_t)(min((int64_t)row, m - 1 - m0) * g.lda) + (uint32_t)(chunk * 16);
  }
#pragma unroll
  for (int i = 0; i < C::kBLoads; ++i) {
    const int sl = 64 * (i * C::kWaves + wv) + lane, row = sl >> 3, chunk = (sl & 7) ^ swz_key(row);
    off[C::kALoads + i] = (uint32_t)(min((int64_t)row, n - 1 - n0) * g.ldb) + (uint32_t)(chunk * 16);
  }
  const uint32_t sa_off = 4u * (uint32_t)min((int64_t)(64 * wv + lane), m - 1 - m0);
  // B: with 1x128 exponents every wave copies one block scale into its own slot (waves
  // 2, 3 repeat those of waves 0, 1), so that no copy depends on a wave-dependent
  // branch; with group 32 each wave copies the words of 64 of the tile's columns
  const int64_t sb_blk = min((int64_t)(n0 >> 7) + (wv & 1), nbl - 1);
  const uint32_t sb_off = 4u * (uint32_t)min((int64_t)(64 * wv + lane), n - 1 - n0);
  const uint32_t *sa = reinterpret_cast<const uint32_t *>(g.sa);
  const uint32_t *sbw = reinterpret_cast<const uint32_t *>(g.sb);
  auto copy_one = [&](int c, int kb, uint8_t *st) {
    if (c < C::kALoads)
      load_lds16(g.A + m0 * g.lda + (int64_t)kb * kBK, off[c], st + 1024 * (c * C::kWaves + wv));
    else
      load_lds16(g.B + n0 * g.ldb + (int64_t)kb * kBK, off[c],
                 st + C::kABytes + 1024 * ((c - C::kALoads) * C::kWaves + wv));
  };
  auto copy_scales = [&](int kb, uint8_t *st) {
    const int64_t col = MODE == kWideUePacked ? (kb >> 2) : kb;
    load_lds4(sa + col * g.sa_ld + m0, sa_off, st + C::kSaOff + 256 * wv);
    if constexpr (G32)
      load_lds4(sbw + (int64_t)kb * g.sb_ld + n0, sb_off, st + C::kSbOff + 256 * wv);
    else
      load_lds4(g.sb + sb_blk * g.sb_ld + kb, 0u, st + C::kSbOff + 256 * wv);
  };

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  const int r32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int c = 0; c < C::kALoads + C::kBLoads; ++c) copy_one(c, 0, smem);
  copy_scales(0, smem);
  for (int kb = 0; kb < KB; ++kb) {
    // block kb has landed (own copies, then everyone's), and every wave is done
    // reading block kb-1's stage, which the copies below refill
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const uint8_t *st = smem + (kb & 1) * C::kStageBytes;
    uint8_t *nst = smem + ((kb + 1) & 1) * C::kStageBytes;
    const int kn = min(kb + 1, KB - 1);
    // exponent words of the lane's rows (A) and columns (B, group 32) or B's block
    // scale; the byte is bits 30-23 of an fp32 2^e, byte kb % 4 of a packed 1x128
    // word, or byte 2s + hh of a group-32 word (MFMA s, below)
    uint32_t wa[4], wb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      wa[i] = *reinterpret_cast<const uint32_t *>(st + C::kSaOff + 4 * (wm + 32 * i + r32));
      wb[i] = G32 ? *reinterpret_cast<const uint32_t *>(st + C::kSbOff + 4 * (wn + 32 * i + r32))
                  : *reinterpret_cast<const uint32_t *>(st + C::kSbOff + 256 * (wn >> 7));
    }
    // A: group-32 byte, byte kb % 4 of a packed 1x128 word, or an fp32 2^e; B: group-32
    // byte, or its block's fp32 2^e in both 1x128 modes
    auto ex_a = [&](uint32_t w, int s) {
      const int sh = G32 ? 8 * (2 * s + hh) : MODE == kWideUePacked ? 8 * (kb & 3) : 23;
      return (int)((w >> sh) & 0xFFu);
    };
    auto ex_b = [&](uint32_t w, int s) { return (int)((w >> (G32 ? 8 * (2 * s + hh) : 23)) & 0xFFu); };
    auto fr = [&](const uint8_t *tile, int row, int s) {
      return G32 ? frag32_g32(tile, row, hh, s) : frag32(tile, row, hh, s);
    };
    v8i af[2][4], bf[2][4];
    af[0][0] = fr(st, wm + r32, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) bf[0][i] = fr(st + C::kABytes, wn + 32 * i + r32, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        // snake order over the 4x4 tiles: each MFMA needs at most one new fragment
        const int mi = q >> 2, ni = (mi & 1) ? 3 - (q & 3) : (q & 3);
        // first operand B (its column's or block's exponent), second A (its row's)
        acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bf[s][ni], af[s][mi], acc[mi][ni], 0, 0, 0,
                                                                      ex_b(wb[ni], s), 0, ex_a(wa[mi], s));
        if (s == 0) {
          // this half's A fragments 1-3, then the other half's fragments
          if (q < 3) af[0][q + 1] = fr(st, wm + 32 * (q + 1) + r32, 0);
          else if (q < 7) af[1][q - 3] = fr(st, wm + 32 * (q - 3) + r32, 1);
          else if (q < 11) bf[1][q - 7] = fr(st + C::kABytes, wn + 32 * (q - 7) + r32, 1);
          copy_one(q, kn, nst);   // one copy of the next block per MFMA
        } else if (q == 0) {
          copy_scales(kn, nst);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // no copy in flight at exit

  // epilogue: lane (r32, hh) of tile (mi, ni) holds row r32 and columns 8q + 4hh .. +3
  // for q = 0..3 (values 4q .. 4q+3)
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int64_t i = m0 + wm + 32 * mi + r32;
    if (i >= m) continue;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int64_t j = n0 + wn + 32 * ni + 8 * gq + 4 * hh;
        if (j >= n) continue;
        const v4f v = {acc[mi][ni][4 * gq], acc[mi][ni][4 * gq + 1], acc[mi][ni][4 * gq + 2], acc[mi][ni][4 * gq + 3]};
        store_bf16x4(reinterpret_cast<uint16_t *>(g.D) + i * g.ldd + j, v, n - j);
      }
  }
}

}  // namespace

bool gemm_wide_fits(int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldb) {
  // one or two rounds of 256x256 tiles.  Measured on MI355X against the 128x128
  // scaled-MFMA kernel, same process: 8192x4096x7168 (512 tiles) 200 vs 213 us,
  // 4096x7168x7168 (448) 177 vs 197, 4096x4096x7168 (256) 102 vs 109.  With more
  // rounds the 128x128 kernel's first-round B prefetch and second workgroup per CU
  // win where B is cold: 8192x7168x4096 (896 tiles) as dgrad in the linear step took
  // 246 us against 233 (227 vs 230 isolated).
  // A copy's in-tile offset reaches 255 rows times the leading dimension; below 2^23 it
  // stays under 2^31, as in the 128x128 kernels, whose results are the same
  if (lda >= (int64_t)1 << 23 || ldb >= (int64_t)1 << 23) return false;
  const int64_t tiles = ((m + 255) / 256) * ((n + 255) / 256);
  return tiles >= 256 && tiles <= 512 && k / kBK >= 8;
}

hipError_t launch_gemm_wide(const GemmArgs &a, hipStream_t st) {
  const int tiles_m = (int)((a.m + WideCfg::kBM - 1) / WideCfg::kBM);
  const int tiles_n = (int)((a.n + WideCfg::kBN - 1) / WideCfg::kBN);
  const int per_xcd = (tiles_m * tiles_n + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds));
  if (a.ue_gran == 32)
    hipLaunchKernelGGL((gemm_wide_kernel<kWideG32>), grid, dim3(WideCfg::kThreads), 0, st, a, tiles_m, tiles_n);
  else if (a.sa_fmt == kSfPackedUe8m0)
    hipLaunchKernelGGL((gemm_wide_kernel<kWideUePacked>), grid, dim3(WideCfg::kThreads), 0, st, a, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_wide_kernel<kWideUeFloat>), grid, dim3(WideCfg::kThreads), 0, st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace fgfp8
