// launch.h -- internal interface between the C ABI (abi.hip) and the kernel
// files of libfgfp8.  Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgfp8 {

enum : int { kInBf16 = 0, kInFp32 = 1 };
enum : int { kSfFp32 = 0, kSfUe8m0 = 1, kSfPackedUe8m0 = 2 };

struct CastTokenArgs {
  const void *x;
  int x_dtype;
  int64_t rows, cols, x_stride_row, x_stride_col;
  int gran_k, sf_fmt;
  uint8_t *q;
  int64_t q_ld;
  void *sf;
  int64_t sf_stride_row, sf_stride_group;
};

struct CastBlockArgs {
  const void *x;
  int x_dtype;
  int64_t rows, cols, x_ld;
  int sf_fmt;
  uint8_t *q;
  int64_t q_ld;
  float *sf;
  int64_t sf_ld;
  uint8_t *qT;
  int64_t qT_ld;
  float *sfT;
  int64_t sfT_ld;
};

// Dual-orientation per-token cast (bf16 or fp32 input, group 32 or 128, fp32,
// UE8M0 or packed-UE8M0 scales).
struct CastDualArgs {
  const void *x;
  int x_dtype;
  int64_t rows, cols, x_ld;
  int gran_k, sf_fmt;
  uint8_t *q;
  int64_t q_ld;
  void *sf;
  int64_t sf_stride_row, sf_stride_group;
  uint8_t *qT;
  int64_t qT_ld;
  void *sfT;
  int64_t sfT_stride_row, sfT_stride_group;
};

// One GEMM problem.  wgrad == false: D bf16, sb one scale per 128x128 block
// ((nb, kb) at sb[nb*sb_ld + kb]).  wgrad == true: D fp32 accumulated,
// sb one scale per row and K block ((j, kb) at sb[kb*sb_ld + j]).
struct GemmArgs {
  const uint8_t *A;
  int64_t lda;
  const void *sa;
  int sa_fmt;
  int64_t sa_ld;
  const uint8_t *B;
  int64_t ldb;
  const float *sb;
  int64_t sb_ld;
  void *D;
  int64_t ldd;
  int64_t m, n, k;
  bool wgrad;
  // m-grouped contiguous layout (forward only): row i uses expert m_idx[i]
  // (-1 = padding, not written); expert e's B at B + e*b_estride and its
  // scales at sb + e*sb_estride.  m_idx == nullptr: a plain GEMM.
  const int32_t *m_idx = nullptr;
  int64_t num_experts = 0, b_estride = 0, sb_estride = 0;
  // Per-token cast of the bf16 output fused into the epilogue (forward only):
  // q [m, n] E4M3 (q_ld) and one scale per row and 128-column group at
  // cq_sf[i*cq_s_row + g*cq_s_grp]; cq_fmt kSfFp32 or kSfUe8m0.  D may then be
  // nullptr (the bf16 output is not stored).  q == nullptr: no fused cast.
  uint8_t *q = nullptr;
  int64_t q_ld = 0;
  float *cq_sf = nullptr;
  int64_t cq_s_row = 0, cq_s_grp = 0;
  int cq_fmt = 0;
  // Scaled-MFMA kernel (launch_gemm_g32): group size of the UE8M0 exponents, 32
  // (packed words) or 128 (wgrad only: packed words, or fp32 2^e values when
  // sa_fmt is kSfUe8m0).
  int ue_gran = 32;
  // Workgroups (blockIdx.x below this) that first read all of B through the
  // caches, so that later rounds of tiles find it in the MALL; 0: none.
  int b_prefetch_wgs = 0;
  // K-sliced 128x128 tiles (split-K entry point, m > 64): the fp32 partial sums
  // of slice s of tile t go to slot t*slices + s of part (64 KB each).
  float *part = nullptr;
};

hipError_t launch_cast_per_token(const CastTokenArgs &a, hipStream_t st);
hipError_t launch_cast_per_block(const CastBlockArgs &a, hipStream_t st);
hipError_t launch_cast_dual(const CastDualArgs &a, hipStream_t st);
hipError_t launch_gemm(const GemmArgs &a, hipStream_t st);

// Split-K GEMM (bf16 output).  m <= 64: stream-K over 128-column tiles x K blocks,
// workspace 2*grid slots of 16*ceil(m/16) x 128 fp32 partial sums.  m > 64:
// 128x128 tiles with K cut into `slices` consecutive ranges, one workgroup each,
// workspace tiles*slices slots of 128x128 fp32 (slices == 1: the plain kernel,
// no workspace).
constexpr int64_t kStreamKSlots = 256;   // workgroups the plan aims at (one per CU)
struct SplitKPlan {
  int64_t tiles_n, units, upw, grid, workspace_bytes;
  int64_t tiles_m = 0, slices = 0;
};
SplitKPlan splitk_plan(int64_t m, int64_t n, int64_t k);
hipError_t launch_gemm_splitk(const GemmArgs &a, void *ws, const SplitKPlan &p, hipStream_t st);
// UE8M0 group-32 recipe: sa and sb are packed words (one per row and 128-K block,
// MN-major: (i, kb) at sa[kb*sa_ld + i], (j, kb) at sb[kb*sb_ld + j]).
hipError_t launch_gemm_g32(const GemmArgs &a, hipStream_t st);

}  // namespace fgfp8
