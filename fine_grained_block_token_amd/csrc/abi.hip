// abi.hip -- the extern "C" entry points of libfgfp8.so (declared in
// include/fgfp8.h): host-side argument validation, the gfx950 device check,
// and the launch on the caller's stream.  Every check runs before any HIP
// call that could launch work, so an invalid call writes nothing.
#include <atomic>
#include <cstring>

#include "fgfp8.h"
#include "gemm_wide.h"
#include "launch.h"

namespace {

using fgfp8::kInBf16;
using fgfp8::kInFp32;
using fgfp8::kSfFp32;
using fgfp8::kSfPackedUe8m0;
using fgfp8::kSfUe8m0;

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// 0 = not yet checked, 1 = gfx950, -1 = something else
std::atomic<int> g_device_state[64];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FGFP8_EDEVICE;
  if (dev >= 64) return FGFP8_EDEVICE;
  int s = g_device_state[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FGFP8_EDEVICE;
    s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_device_state[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? FGFP8_OK : FGFP8_EDEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? FGFP8_OK : FGFP8_ELAUNCH; }

// The partial sums of gemm_fp8_nt_bf16_splitk_noalloc: one copy of this array per
// GPU, allocated by the runtime when the library's code object is loaded there and
// held until the process ends.  Host code never uses the name itself (on the host it
// is only a stand-in): the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) uint8_t scratch[FGFP8_SCRATCH_BYTES];

std::atomic<void *> g_scratch_ptr[64];

// Device address of `scratch` on device `dev` (the current device), looked up once.
void *scratch_ptr(int dev) {
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

int cast_per_token(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t x_stride_row,
                   int64_t x_stride_col, int gran_k, int sf_fmt, uint8_t *q, int64_t q_ld, void *sf,
                   int64_t sf_stride_row, int64_t sf_stride_group, void *stream) {
  if (x_dtype != kInBf16 && x_dtype != kInFp32) return FGFP8_EINVAL;
  if (gran_k != 32 && gran_k != 128) return FGFP8_EINVAL;
  if (sf_fmt != kSfFp32 && sf_fmt != kSfUe8m0 && sf_fmt != kSfPackedUe8m0) return FGFP8_EINVAL;
  if (rows < 0 || cols < 0) return FGFP8_EINVAL;
  if (rows == 0 || cols == 0) return FGFP8_OK;
  if (!x || !q || !sf) return FGFP8_EINVAL;
  const int64_t es = x_dtype == kInBf16 ? 2 : 4;
  bool transposed;
  if (x_stride_col == 1 && x_stride_row >= cols) {
    transposed = false;
    if ((x_stride_row * es) % 16 != 0 && rows > 1) return FGFP8_EINVAL;
  } else if (x_stride_row == 1 && x_stride_col >= rows) {
    transposed = true;
    if ((x_stride_col * es) % 16 != 0) return FGFP8_EINVAL;
    // one workgroup per 64 rows x 128 columns, column tiles along the grid's y
    if (cdiv(cols, 128) > FGFP8_MAX_CAST_COL_TILES || cdiv(rows, 64) > FGFP8_MAX_CAST_TILES) return FGFP8_EINVAL;
  } else {
    return FGFP8_EINVAL;
  }
  if (!aligned(x, 16)) return FGFP8_EINVAL;
  const int64_t qa = transposed ? 16 : 8;
  if (!aligned(q, qa) || q_ld < cols || q_ld % qa != 0) return FGFP8_EINVAL;
  if (!aligned(sf, 4)) return FGFP8_EINVAL;
  const int64_t groups = cdiv(cols, gran_k);
  const int64_t units = sf_fmt == kSfPackedUe8m0 ? cdiv(groups, 4) : groups;
  const bool row_major_sf = sf_stride_group == 1 && sf_stride_row >= units;
  const bool mn_major_sf = sf_stride_row == 1 && sf_stride_group >= rows;
  if (!row_major_sf && !mn_major_sf) return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::CastTokenArgs a{x, x_dtype, rows, cols, x_stride_row, x_stride_col, gran_k, sf_fmt,
                         q, q_ld, sf, sf_stride_row, sf_stride_group};
  return launched(fgfp8::launch_cast_per_token(a, static_cast<hipStream_t>(stream)));
}

int cast_per_block(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t x_ld, int sf_fmt,
                   uint8_t *q, int64_t q_ld, float *sf, int64_t sf_ld, uint8_t *qT, int64_t qT_ld,
                   float *sfT, int64_t sfT_ld, void *stream) {
  if (x_dtype != kInBf16 && x_dtype != kInFp32) return FGFP8_EINVAL;
  if (sf_fmt != kSfFp32 && sf_fmt != kSfUe8m0) return FGFP8_EINVAL;
  if (rows < 0 || cols < 0) return FGFP8_EINVAL;
  if ((qT == nullptr) != (sfT == nullptr)) return FGFP8_EINVAL;
  if (rows == 0 || cols == 0) return FGFP8_OK;
  if (!x || !q || !sf) return FGFP8_EINVAL;
  const int64_t es = x_dtype == kInBf16 ? 2 : 4;
  if (!aligned(x, 16) || x_ld < cols || (x_ld * es) % 16 != 0) return FGFP8_EINVAL;
  if (!aligned(q, 8) || q_ld < cols || q_ld % 8 != 0) return FGFP8_EINVAL;
  if (!aligned(sf, 4) || sf_ld < cdiv(cols, 128)) return FGFP8_EINVAL;
  if (qT) {
    if (!aligned(qT, 16) || qT_ld < rows || qT_ld % 16 != 0) return FGFP8_EINVAL;
    if (!aligned(sfT, 4) || sfT_ld < cdiv(rows, 128)) return FGFP8_EINVAL;
  }
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::CastBlockArgs a{x, x_dtype, rows, cols, x_ld, sf_fmt, q, q_ld, sf, sf_ld, qT, qT_ld, sfT, sfT_ld};
  return launched(fgfp8::launch_cast_per_block(a, static_cast<hipStream_t>(stream)));
}

// (r, g) -> r*s_row + g*s_grp is one of the two layouts the kernels write:
// row-major (s_grp == 1, s_row >= groups) or MN-major (s_row == 1, s_grp >= rows).
static bool scale_layout_ok(int64_t rows, int64_t groups, int64_t s_row, int64_t s_grp) {
  return (s_grp == 1 && s_row >= groups) || (s_row == 1 && s_grp >= rows);
}

int cast_per_token_dual(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t x_ld, int gran_k,
                        int sf_fmt, uint8_t *q, int64_t q_ld, void *sf, int64_t sf_stride_row,
                        int64_t sf_stride_group, uint8_t *qT, int64_t qT_ld, void *sfT, int64_t sfT_stride_row,
                        int64_t sfT_stride_group, void *stream) {
  if (x_dtype != kInBf16 && x_dtype != kInFp32) return FGFP8_EINVAL;
  if (gran_k != 32 && gran_k != 128) return FGFP8_EINVAL;
  if (sf_fmt != kSfFp32 && sf_fmt != kSfUe8m0 && sf_fmt != kSfPackedUe8m0) return FGFP8_EINVAL;
  if (rows < 0 || cols < 0) return FGFP8_EINVAL;
  if (rows == 0 || cols == 0) return FGFP8_OK;
  if (!x || !q || !sf || !qT || !sfT) return FGFP8_EINVAL;
  const int64_t es = x_dtype == kInBf16 ? 2 : 4;
  if (!aligned(x, 16) || x_ld < cols || (x_ld * es) % 16 != 0) return FGFP8_EINVAL;
  if (!aligned(q, 8) || q_ld < cols || q_ld % 8 != 0) return FGFP8_EINVAL;
  if (!aligned(qT, 16) || qT_ld < rows || qT_ld % 16 != 0) return FGFP8_EINVAL;
  if (!aligned(sf, 4) || !aligned(sfT, 4)) return FGFP8_EINVAL;
  // scale units per row: groups, or packed words of four groups
  const bool packed = sf_fmt == kSfPackedUe8m0;
  const int64_t units = packed ? cdiv(cdiv(cols, gran_k), 4) : cdiv(cols, gran_k);
  const int64_t unitsT = packed ? cdiv(cdiv(rows, gran_k), 4) : cdiv(rows, gran_k);
  if (!scale_layout_ok(rows, units, sf_stride_row, sf_stride_group)) return FGFP8_EINVAL;
  if (!scale_layout_ok(cols, unitsT, sfT_stride_row, sfT_stride_group)) return FGFP8_EINVAL;
  // one workgroup of 256 threads per 128x128 tile: at most 2^24 tiles in a launch
  if (rows > FGFP8_MAX_CAST_TILES * 128 || cols > FGFP8_MAX_CAST_TILES * 128 ||
      cdiv(rows, 128) * cdiv(cols, 128) > FGFP8_MAX_CAST_TILES)
    return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::CastDualArgs a{x, x_dtype, rows, cols, x_ld, gran_k, sf_fmt, q, q_ld, sf, sf_stride_row,
                        sf_stride_group, qT, qT_ld, sfT, sfT_stride_row, sfT_stride_group};
  return launched(fgfp8::launch_cast_dual(a, static_cast<hipStream_t>(stream)));
}

// Size limits of the GEMMs (FGFP8_MAX_GEMM_TILES, FGFP8_MAX_GEMM_N in fgfp8.h).
constexpr int64_t kMaxTiles = FGFP8_MAX_GEMM_TILES, kMaxN = FGFP8_MAX_GEMM_N, kMaxMN = kMaxTiles * 128;

static int check_gemm_common(const uint8_t *A, int64_t lda, const void *sa, int64_t sa_ld, const uint8_t *B,
                             int64_t ldb, const float *sb, const void *D, int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k <= 0 || k % 128 != 0) return FGFP8_EINVAL;
  if (m == 0 || n == 0) return FGFP8_OK;
  if (!A || !B || !sa || !sb || !D) return FGFP8_EINVAL;
  if (!aligned(A, 16) || lda < k || lda % 16 != 0) return FGFP8_EINVAL;
  if (!aligned(B, 16) || ldb < k || ldb % 16 != 0) return FGFP8_EINVAL;
  if (!aligned(sa, 4) || !aligned(sb, 4) || sa_ld < m) return FGFP8_EINVAL;
  if (lda >= (int64_t)1 << 24 || ldb >= (int64_t)1 << 24) return FGFP8_EINVAL;  // 32-bit in-tile offsets
  // grid limits: tile counts stay in 32-bit ints and every launch within 2^32 work-items
  if (m > kMaxMN || n > kMaxN || cdiv(m, 128) * cdiv(n, 128) > kMaxTiles) return FGFP8_EINVAL;
  return 1;  // proceed
}

int gemm_fp8_nt_bf16(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt, int64_t sa_ld,
                     const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld, uint16_t *D, int64_t ldd,
                     int64_t m, int64_t n, int64_t k, void *stream) {
  if (sa_fmt != kSfFp32 && sa_fmt != kSfUe8m0 && sa_fmt != kSfPackedUe8m0) return FGFP8_EINVAL;
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, sb, D, m, n, k);
  if (c != 1) return c;
  if (sb_ld < k / 128) return FGFP8_EINVAL;
  if (!aligned(D, 16) || ldd < n || ldd % 8 != 0) return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::GemmArgs a{A, lda, sa, sa_fmt, sa_ld, B, ldb, sb, sb_ld, D, ldd, m, n, k, false};
  return launched(fgfp8::launch_gemm(a, static_cast<hipStream_t>(stream)));
}

// Limits of the split-K plans: stream-K (m <= 64) indexes units in 32 bits and runs
// up to 4 fix-up workgroups per 128-column tile; K slices (m > 64) share
// gemm_fp8_nt_bf16's tile-count limit.
static bool splitk_fits(int64_t m, int64_t n, int64_t k) {
  if (m > kMaxMN || n > kMaxN || cdiv(m, 128) * cdiv(n, 128) > kMaxTiles) return false;
  if (m > 64) return true;
  return k / 128 <= 0x7FFFFFF0 && cdiv(n, 128) * (k / 128) <= 0x7FFFFFF0;
}

int64_t gemm_fp8_nt_bf16_splitk_workspace(int64_t m, int64_t n, int64_t k) {
  if (m < 0 || n < 0 || k <= 0 || k % 128 != 0) return FGFP8_EINVAL;
  if (m == 0 || n == 0) return 0;
  if (!splitk_fits(m, n, k)) return FGFP8_EINVAL;
  return fgfp8::splitk_plan(m, n, k).workspace_bytes;
}

int gemm_fp8_nt_bf16_splitk(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt, int64_t sa_ld,
                            const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld, uint16_t *D, int64_t ldd,
                            int64_t m, int64_t n, int64_t k, void *workspace, int64_t workspace_bytes,
                            void *stream) {
  if (sa_fmt != kSfFp32 && sa_fmt != kSfUe8m0 && sa_fmt != kSfPackedUe8m0) return FGFP8_EINVAL;
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, sb, D, m, n, k);
  if (c != 1) return c;
  if (sb_ld < k / 128) return FGFP8_EINVAL;
  if (!aligned(D, 16) || ldd < n || ldd % 8 != 0) return FGFP8_EINVAL;
  if (!splitk_fits(m, n, k)) return FGFP8_EINVAL;
  const fgfp8::SplitKPlan plan = fgfp8::splitk_plan(m, n, k);
  if (plan.workspace_bytes > 0 && (!workspace || !aligned(workspace, 16) || workspace_bytes < plan.workspace_bytes))
    return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::GemmArgs a{A, lda, sa, sa_fmt, sa_ld, B, ldb, sb, sb_ld, D, ldd, m, n, k, false};
  return launched(fgfp8::launch_gemm_splitk(a, workspace, plan, static_cast<hipStream_t>(stream)));
}

int gemm_fp8_nt_bf16_splitk_noalloc(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt, int64_t sa_ld,
                                    const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld, uint16_t *D,
                                    int64_t ldd, int64_t m, int64_t n, int64_t k, void *stream) {
  if (sa_fmt != kSfFp32 && sa_fmt != kSfUe8m0 && sa_fmt != kSfPackedUe8m0) return FGFP8_EINVAL;
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, sb, D, m, n, k);
  if (c != 1) return c;
  if (sb_ld < k / 128) return FGFP8_EINVAL;
  if (!aligned(D, 16) || ldd < n || ldd % 8 != 0) return FGFP8_EINVAL;
  if (!splitk_fits(m, n, k)) return FGFP8_EINVAL;
  const fgfp8::SplitKPlan plan = fgfp8::splitk_plan(m, n, k);
  if (plan.workspace_bytes > FGFP8_SCRATCH_BYTES) return FGFP8_ESCRATCH;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  int d = -1;
  if (hipGetDevice(&d) != hipSuccess || d < 0 || d >= 64) return FGFP8_EDEVICE;
  void *ws = scratch_ptr(d);
  if (!ws) return FGFP8_EDEVICE;
  fgfp8::GemmArgs a{A, lda, sa, sa_fmt, sa_ld, B, ldb, sb, sb_ld, D, ldd, m, n, k, false};
  return launched(fgfp8::launch_gemm_splitk(a, ws, plan, static_cast<hipStream_t>(stream)));
}

int gemm_fp8_nt_bf16_cast(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt, int64_t sa_ld,
                          const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld, uint16_t *D, int64_t ldd,
                          int q_sf_fmt, uint8_t *q, int64_t q_ld, float *q_sf, int64_t q_sf_stride_row,
                          int64_t q_sf_stride_group, int64_t m, int64_t n, int64_t k, void *stream) {
  if (sa_fmt != kSfFp32 && sa_fmt != kSfUe8m0 && sa_fmt != kSfPackedUe8m0) return FGFP8_EINVAL;
  if (q_sf_fmt != kSfFp32 && q_sf_fmt != kSfUe8m0) return FGFP8_EINVAL;
  // D is optional here: check_gemm_common wants a pointer, so hand it q
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, sb, q, m, n, k);
  if (c != 1) return c;
  if (sb_ld < k / 128) return FGFP8_EINVAL;
  if (D && (!aligned(D, 16) || ldd < n || ldd % 8 != 0)) return FGFP8_EINVAL;
  if (!aligned(q, 4) || q_ld < n || q_ld % 4 != 0) return FGFP8_EINVAL;
  if (!q_sf || !aligned(q_sf, 4)) return FGFP8_EINVAL;
  if (!scale_layout_ok(m, cdiv(n, 128), q_sf_stride_row, q_sf_stride_group)) return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::GemmArgs a{A, lda, sa, sa_fmt, sa_ld, B, ldb, sb, sb_ld, D, ldd, m, n, k, false};
  a.q = q;
  a.q_ld = q_ld;
  a.cq_sf = q_sf;
  a.cq_s_row = q_sf_stride_row;
  a.cq_s_grp = q_sf_stride_group;
  a.cq_fmt = q_sf_fmt;
  return launched(fgfp8::launch_gemm(a, static_cast<hipStream_t>(stream)));
}

int gemm_fp8_nt_bf16_ue8m0_g32(const uint8_t *A, int64_t lda, const uint32_t *sa, int64_t sa_ld,
                               const uint8_t *B, int64_t ldb, const uint32_t *sb, int64_t sb_ld, uint16_t *D,
                               int64_t ldd, int64_t m, int64_t n, int64_t k, void *stream) {
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, reinterpret_cast<const float *>(sb), D, m, n, k);
  if (c != 1) return c;
  if (sb_ld < n) return FGFP8_EINVAL;
  if (!aligned(D, 16) || ldd < n || ldd % 8 != 0) return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::GemmArgs a{A, lda, sa, kSfPackedUe8m0, sa_ld, B, ldb, reinterpret_cast<const float *>(sb), sb_ld,
                    D, ldd, m, n, k, false};
  if (fgfp8::gemm_wide_fits(m, n, k, lda, ldb)) return launched(fgfp8::launch_gemm_wide(a, static_cast<hipStream_t>(stream)));
  return launched(fgfp8::launch_gemm_g32(a, static_cast<hipStream_t>(stream)));
}

int gemm_fp8_nt_bf16_ue8m0(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt, int64_t sa_ld,
                           const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld, uint16_t *D, int64_t ldd,
                           int64_t m, int64_t n, int64_t k, void *stream) {
  if (sa_fmt != kSfUe8m0 && sa_fmt != kSfPackedUe8m0) return FGFP8_EINVAL;
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, sb, D, m, n, k);
  if (c != 1) return c;
  if (sb_ld < k / 128) return FGFP8_EINVAL;
  if (!aligned(D, 16) || ldd < n || ldd % 8 != 0) return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::GemmArgs a{A, lda, sa, sa_fmt, sa_ld, B, ldb, sb, sb_ld, D, ldd, m, n, k, false};
  a.ue_gran = 128;
  // one or two full rounds of 256x256 tiles: the wide kernel (same bits, fewer copied
  // bytes per flop); otherwise the 128x128 kernel fills the part better
  if (fgfp8::gemm_wide_fits(m, n, k, lda, ldb)) return launched(fgfp8::launch_gemm_wide(a, static_cast<hipStream_t>(stream)));
  return launched(fgfp8::launch_gemm_g32(a, static_cast<hipStream_t>(stream)));
}

int wgrad_gemm_fp8_nt_fp32_ue8m0(const uint8_t *A, int64_t lda, const void *sa, int sf_fmt, int64_t sa_ld,
                                 const uint8_t *B, int64_t ldb, const void *sb, int64_t sb_ld, float *D, int64_t ldd,
                                 int64_t m, int64_t n, int64_t k, void *stream) {
  if (sf_fmt != kSfUe8m0 && sf_fmt != kSfPackedUe8m0) return FGFP8_EINVAL;
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, reinterpret_cast<const float *>(sb), D, m, n, k);
  if (c != 1) return c;
  if (sb_ld < n) return FGFP8_EINVAL;
  if (!aligned(D, 16) || ldd < n || ldd % 4 != 0) return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::GemmArgs a{A, lda, sa, sf_fmt, sa_ld, B, ldb, reinterpret_cast<const float *>(sb), sb_ld,
                    D, ldd, m, n, k, true};
  a.ue_gran = 128;
  return launched(fgfp8::launch_gemm_g32(a, static_cast<hipStream_t>(stream)));
}

int wgrad_gemm_fp8_nt_fp32_ue8m0_g32(const uint8_t *A, int64_t lda, const uint32_t *sa, int64_t sa_ld,
                                     const uint8_t *B, int64_t ldb, const uint32_t *sb, int64_t sb_ld, float *D,
                                     int64_t ldd, int64_t m, int64_t n, int64_t k, void *stream) {
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, reinterpret_cast<const float *>(sb), D, m, n, k);
  if (c != 1) return c;
  if (sb_ld < n) return FGFP8_EINVAL;
  if (!aligned(D, 16) || ldd < n || ldd % 4 != 0) return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::GemmArgs a{A, lda, sa, kSfPackedUe8m0, sa_ld, B, ldb, reinterpret_cast<const float *>(sb), sb_ld,
                    D, ldd, m, n, k, true};
  return launched(fgfp8::launch_gemm_g32(a, static_cast<hipStream_t>(stream)));
}

int m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(const uint8_t *A, int64_t lda, const uint32_t *sa,
                                                    int64_t sa_ld, const uint8_t *B, int64_t ldb,
                                                    int64_t b_expert_stride, const uint32_t *sb, int64_t sb_ld,
                                                    int64_t sb_expert_stride, const int32_t *m_indices,
                                                    int64_t num_experts, uint16_t *D, int64_t ldd, int64_t m,
                                                    int64_t n, int64_t k, void *stream) {
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, reinterpret_cast<const float *>(sb), D, m, n, k);
  if (c != 1) return c;
  if (sb_ld < n) return FGFP8_EINVAL;
  if (!aligned(D, 16) || ldd < n || ldd % 8 != 0) return FGFP8_EINVAL;
  if (num_experts < 1 || num_experts > 0x7FFFFFFF || !m_indices || !aligned(m_indices, 4)) return FGFP8_EINVAL;
  if (b_expert_stride < (n - 1) * ldb + k || b_expert_stride % 16 != 0) return FGFP8_EINVAL;
  if (sb_expert_stride < (k / 128 - 1) * sb_ld + n) return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::GemmArgs a{A, lda, sa, kSfPackedUe8m0, sa_ld, B, ldb, reinterpret_cast<const float *>(sb), sb_ld,
                    D, ldd, m, n, k, false};
  a.m_idx = m_indices;
  a.num_experts = num_experts;
  a.b_estride = b_expert_stride;
  a.sb_estride = sb_expert_stride;
  return launched(fgfp8::launch_gemm_g32(a, static_cast<hipStream_t>(stream)));
}

int m_grouped_gemm_fp8_nt_bf16_contiguous(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt,
                                          int64_t sa_ld, const uint8_t *B, int64_t ldb, int64_t b_expert_stride,
                                          const float *sb, int64_t sb_ld, int64_t sb_expert_stride,
                                          const int32_t *m_indices, int64_t num_experts, uint16_t *D,
                                          int64_t ldd, int64_t m, int64_t n, int64_t k, void *stream) {
  if (sa_fmt != kSfFp32 && sa_fmt != kSfUe8m0 && sa_fmt != kSfPackedUe8m0) return FGFP8_EINVAL;
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, sb, D, m, n, k);
  if (c != 1) return c;
  if (sb_ld < k / 128) return FGFP8_EINVAL;
  if (!aligned(D, 16) || ldd < n || ldd % 8 != 0) return FGFP8_EINVAL;
  if (num_experts < 1 || num_experts > 0x7FFFFFFF || !m_indices || !aligned(m_indices, 4)) return FGFP8_EINVAL;
  // experts' weights must not overlap: B[e] is [n, k] with leading dimension ldb
  if (b_expert_stride < (n - 1) * ldb + k || b_expert_stride % 16 != 0) return FGFP8_EINVAL;
  if (sb_expert_stride < (cdiv(n, 128) - 1) * sb_ld + k / 128) return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::GemmArgs a{A, lda, sa, sa_fmt, sa_ld, B, ldb, sb, sb_ld, D, ldd, m, n, k, false};
  a.m_idx = m_indices;
  a.num_experts = num_experts;
  a.b_estride = b_expert_stride;
  a.sb_estride = sb_expert_stride;
  return launched(fgfp8::launch_gemm(a, static_cast<hipStream_t>(stream)));
}

int wgrad_gemm_fp8_nt_fp32(const uint8_t *A, int64_t lda, const float *sa, int64_t sa_ld, const uint8_t *B,
                           int64_t ldb, const float *sb, int64_t sb_ld, float *D, int64_t ldd, int64_t m,
                           int64_t n, int64_t k, void *stream) {
  const int c = check_gemm_common(A, lda, sa, sa_ld, B, ldb, sb, D, m, n, k);
  if (c != 1) return c;
  if (sb_ld < n) return FGFP8_EINVAL;
  if (!aligned(D, 16) || ldd < n || ldd % 4 != 0) return FGFP8_EINVAL;
  const int dev = check_device();
  if (dev != FGFP8_OK) return dev;
  fgfp8::GemmArgs a{A, lda, sa, kSfFp32, sa_ld, B, ldb, sb, sb_ld, D, ldd, m, n, k, true};
  return launched(fgfp8::launch_gemm(a, static_cast<hipStream_t>(stream)));
}

const char *fgfp8_status_string(int status) {
  switch (status) {
    case FGFP8_OK: return "ok";
    case FGFP8_EINVAL: return "invalid argument (nothing launched)";
    case FGFP8_EDEVICE: return "current device is not gfx950";
    case FGFP8_ELAUNCH: return "kernel launch failed";
    case FGFP8_ESCRATCH: return "problem needs more than the 32 MiB static scratch (nothing launched)";
    default: return "unknown status";
  }
}

}  // extern "C"
