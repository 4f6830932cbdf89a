// gemm_wide.h -- the 256x256-tile FP8 GEMM for power-of-two scales (gemm_wide.hip),
// called from the C ABI.  Arguments arrive validated, as for launch_gemm.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.h"

namespace fgfp8 {

// True when launch_gemm_wide is the faster kernel for an m x n x k bf16 GEMM with
// power-of-two scales (UE8M0 1x128 A scales and 128x128 B block scales, or group 32
// on both operands): one or two full rounds of
// 256x256 tiles on a 256-CU part (256 to 512 tiles), at least 8 K blocks, and leading
// dimensions of A and B below 2^23.
bool gemm_wide_fits(int64_t m, int64_t n, int64_t k, int64_t lda, int64_t ldb);

// D = (A * 2^ea)(B * 2^eb)^T, bf16.  a.ue_gran 128: a.sa_fmt kSfUe8m0 (fp32 2^e) or
// kSfPackedUe8m0 (one word per row and four K blocks), MN-major, and a.sb fp32 2^e per
// 128x128 block.  a.ue_gran 32: a.sa and a.sb packed group-32 words, one per row (or
// column) and 128-K block, MN-major.  The same predicate (gemm_wide_fits) for both.
hipError_t launch_gemm_wide(const GemmArgs &a, hipStream_t st);

}  // namespace fgfp8
