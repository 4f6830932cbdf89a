/*
 * fgfp8.h -- C ABI of libfgfp8.so: fine-grained block-scaled FP8 cast and
 * NT GEMM for AMD Instinct MI355X (gfx950).
 *
 * Plain C: pointers, sizes and an opaque stream.  Every pointer named as a
 * tensor below is DEVICE memory owned by the caller; the library allocates
 * nothing at run time and keeps no state beyond a per-device "is this gfx950"
 * check, the runtime's occupancy figures for its persistent cast kernels, and
 * the static device array of gemm_fp8_nt_bf16_splitk_noalloc (32 MiB on each
 * GPU the library is loaded on, held until the process ends).
 * `stream` is a hipStream_t passed as void* (NULL = the default stream).
 * Every call is asynchronous and stream-ordered; none synchronises the host.
 *
 * Return codes (every entry point):
 *   FGFP8_OK (0)        launched (or nothing to do: a zero-sized problem)
 *   FGFP8_EINVAL (-1)   invalid argument, detected on the host before any
 *                       launch: nothing was written
 *   FGFP8_EDEVICE (-2)  the current device is not gfx950 (or no device)
 *   FGFP8_ELAUNCH (-3)  the kernel launch failed (hipGetLastError)
 *   FGFP8_ESCRATCH (-4) gemm_fp8_nt_bf16_splitk_noalloc only: the problem
 *                       needs more than the library's static scratch
 *                       (FGFP8_SCRATCH_BYTES); nothing was written
 * Nothing aborts, throws or prints.
 *
 * Formats.  E4M3 is the OCP FP8 "fn" format (bias 7, largest finite 448, no
 * infinities), one byte per element.  bf16 is the upper half of an fp32.
 * Scale formats:
 *   FGFP8_SF_FP32          fp32 scale = amax / 448
 *   FGFP8_SF_UE8M0         fp32 holding 2^e, the least power of two >= amax/448
 *   FGFP8_SF_PACKED_UE8M0  int32 words; byte b of word w is e + 127 of group
 *                          4w + b (little-endian); unused bytes of the last
 *                          word are 0
 *
 * Sources (web pages, cited by title and section):
 *   "DeepGEMM Essentials: High-Performance FP8 Matrix Multiplication"
 *     (dev.to), Parts 1, 3-6, 8-13, 18;
 *   "[Help] Starter script for nn.Linear for fwd,bwd" (DeepGEMM issue #102):
 *     forward / dgrad / wgrad composition and the RHS scale-row layout;
 *   "deep-gemm: fused per-token FP8 cast in Triton" (kernels-community PR
 *     #1326): cast options, caller-given output views, no host sync.
 */
#ifndef FGFP8_H
#define FGFP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FGFP8_OK 0
#define FGFP8_EINVAL (-1)
#define FGFP8_EDEVICE (-2)
#define FGFP8_ELAUNCH (-3)
#define FGFP8_ESCRATCH (-4)

/* bytes of the static device scratch of gemm_fp8_nt_bf16_splitk_noalloc */
#define FGFP8_SCRATCH_BYTES (32LL << 20)

/* Size limits (beyond them a call returns FGFP8_EINVAL and launches nothing).
 * They keep tile counts in 32-bit integers and every launch within the 2^32
 * work-items of one grid dimension.
 *   GEMMs (every entry point): ceil(m/128) * ceil(n/128) <= FGFP8_MAX_GEMM_TILES
 *     and n <= FGFP8_MAX_GEMM_N.
 *   cast_per_token_dual: ceil(rows/128) * ceil(cols/128) <= FGFP8_MAX_CAST_TILES.
 *   cast_per_token on a transposed view: ceil(rows/64) <= FGFP8_MAX_CAST_TILES
 *     and ceil(cols/128) <= FGFP8_MAX_CAST_COL_TILES. */
#define FGFP8_MAX_GEMM_TILES (1LL << 22)
#define FGFP8_MAX_GEMM_N (1LL << 24)
#define FGFP8_MAX_CAST_TILES (1LL << 24)
#define FGFP8_MAX_CAST_COL_TILES 65535LL

#define FGFP8_IN_BF16 0
#define FGFP8_IN_FP32 1

#define FGFP8_SF_FP32 0
#define FGFP8_SF_UE8M0 1
#define FGFP8_SF_PACKED_UE8M0 2

/*
 * cast_per_token -- per-token (1 x gran_k group) FP8 cast.
 * Defined by "DeepGEMM Essentials", Part 3 (amax per 1x128 group along a
 * row, clamped at 1e-4; scale amax/448; elements times 448/amax rounded to
 * E4M3), with the group 32 / UE8M0 / packed-UE8M0 options and bf16 or fp32
 * input of "deep-gemm: fused per-token FP8 cast in Triton".
 *
 * x          input, x_dtype FGFP8_IN_BF16 or FGFP8_IN_FP32, logical shape
 *            [rows, cols]; element (r, c) at x[r*x_stride_row + c*x_stride_col]
 *            (strides in elements).  Two layouts are accepted:
 *              row-major view:  x_stride_col == 1, x_stride_row >= cols;
 *              transposed view: x_stride_row == 1, x_stride_col >= rows
 *              (the transpose of a row-major [cols, x_stride_col] matrix,
 *              as the wgrad operands are read).
 *            x must be 16-byte aligned and the non-unit stride a multiple of
 *            16 bytes.  A transposed view is also held to the size limits
 *            (FGFP8_MAX_CAST_TILES, FGFP8_MAX_CAST_COL_TILES).
 * gran_k     group size along the columns: 32 or 128.  Groups per row
 *            G = ceil(cols / gran_k); a partial last group takes its amax
 *            over its valid columns only.
 * sf_fmt     FGFP8_SF_FP32, FGFP8_SF_UE8M0 or FGFP8_SF_PACKED_UE8M0.
 * q          E4M3 output [rows, cols], element (r, c) at q[r*q_ld + c];
 *            q 8-byte aligned, q_ld >= cols and a multiple of 8 (row-major
 *            input) or of 16 (transposed input).
 * sf         scales.  fp32 / UE8M0: float (r, g) at
 *            sf[r*sf_stride_row + g*sf_stride_group], g < G.  Packed: int32
 *            word (r, w) at sf[r*sf_stride_row + w*sf_stride_group],
 *            w < ceil(G/4).  Row-major scales: (G or ceil(G/4), 1); the
 *            GEMM's MN-major layout: (1, ld) with ld >= rows.  Strides must
 *            be positive and the (r, g) -> offset map one-to-one.
 * Writes exactly the rows x cols bytes of q and the rows x G scales (or
 * rows x ceil(G/4) words) and nothing else of either buffer.
 * rows == 0 or cols == 0: returns FGFP8_OK and launches nothing.
 */
int cast_per_token(const void *x, int x_dtype, int64_t rows, int64_t cols,
                   int64_t x_stride_row, int64_t x_stride_col,
                   int gran_k, int sf_fmt,
                   uint8_t *q, int64_t q_ld,
                   void *sf, int64_t sf_stride_row, int64_t sf_stride_group,
                   void *stream);

/*
 * cast_per_block -- 128 x 128 block FP8 cast (the RHS / weight operand).
 * Defined by "DeepGEMM Essentials", Part 4 (amax per 128x128 block, same
 * clamp, scale and rounding as the per-token cast).  The optional transposed
 * output is the exact transpose of (q, sf): the block cast commutes with
 * transposition, so it is the dgrad RHS (the transpose of the FP8 weight in
 * the maintainer's pseudo-code of "[Help] Starter script for nn.Linear for
 * fwd,bwd") with no second rounding.
 *
 * x       bf16 or fp32 [rows, cols] row-major, leading dimension x_ld >= cols
 *         (elements); 16-byte aligned, x_ld a multiple of 16 bytes.
 * sf_fmt  FGFP8_SF_FP32 or FGFP8_SF_UE8M0 (fp32 holding 2^e).
 * q       E4M3 [rows, cols], ld q_ld >= cols, multiple of 8; q 8-B aligned.
 * sf      fp32 [ceil(rows/128), ceil(cols/128)], block (bi, bj) at
 *         sf[bi*sf_ld + bj], sf_ld >= ceil(cols/128).
 * qT      NULL, or E4M3 [cols, rows] = q^T, ld qT_ld >= rows, multiple of 16.
 * sfT     NULL iff qT is NULL; fp32 [ceil(cols/128), ceil(rows/128)] = sf^T,
 *         ld sfT_ld >= ceil(rows/128).
 */
int cast_per_block(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t x_ld,
                   int sf_fmt, uint8_t *q, int64_t q_ld, float *sf, int64_t sf_ld,
                   uint8_t *qT, int64_t qT_ld, float *sfT, int64_t sfT_ld,
                   void *stream);

/*
 * cast_per_token_dual -- both per-token casts of one bf16 or fp32 matrix from a single
 * read: the row-wise cast of x [rows, cols] (1 x gran_k groups along cols) and
 * the row-wise cast of its transpose x^T [cols, rows] (1 x gran_k groups along
 * rows).  Each output is bit-identical to the corresponding cast_per_token
 * call with the same gran_k and sf_fmt (on x, and on the transposed view of
 * x).  In an FP8 linear layer the first feeds the forward (or dgrad) GEMM and
 * the second the weight-gradient GEMM, whose K runs over tokens: "[Help]
 * Starter script for nn.Linear for fwd,bwd" (the wgrad line of the
 * maintainer's pseudo-code) and "DeepGEMM Essentials", Part 3 (the group
 * rule); group 32 and the scale formats as in "deep-gemm: fused per-token FP8
 * cast in Triton".  With gran_k = 32 and packed scales it also casts a weight
 * W for the group-32 recipe: q feeds the forward GEMM, qT the dgrad GEMM.
 *
 * x        bf16 (x_dtype FGFP8_IN_BF16) or fp32 (FGFP8_IN_FP32) [rows, cols]
 *          row-major, x_ld >= cols, rows of a multiple of 16 bytes (x_ld a
 *          multiple of 8 bf16 or 4 fp32 elements); 16-byte aligned.
 * gran_k   32 or 128.
 * sf_fmt   FGFP8_SF_FP32, FGFP8_SF_UE8M0 or FGFP8_SF_PACKED_UE8M0.
 * q, sf    as cast_per_token on x: q [rows, cols] (8-byte aligned, q_ld >= cols,
 *          multiple of 8); sf float (r, g) at sf[r*sf_stride_row +
 *          g*sf_stride_group], g < ceil(cols/gran_k), or packed int32 word
 *          (r, w) at the same place, w < ceil(ceil(cols/gran_k)/4);
 *          row-major or MN-major.
 * qT, sfT  as cast_per_token on x^T: qT [cols, rows] (16-byte aligned,
 *          qT_ld >= rows, multiple of 16); sfT (c, g) or (c, w) at
 *          sfT[c*sfT_stride_row + g*sfT_stride_group], g < ceil(rows/gran_k).
 * ceil(rows/128) * ceil(cols/128) <= FGFP8_MAX_CAST_TILES.
 * Writes exactly those elements.  rows == 0 or cols == 0: FGFP8_OK, nothing
 * launched.
 */
int cast_per_token_dual(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t x_ld,
                        int gran_k, int sf_fmt, uint8_t *q, int64_t q_ld,
                        void *sf, int64_t sf_stride_row, int64_t sf_stride_group,
                        uint8_t *qT, int64_t qT_ld,
                        void *sfT, int64_t sfT_stride_row, int64_t sfT_stride_group,
                        void *stream);

/*
 * gemm_fp8_nt_bf16 -- D = (A * sa)(B * sb)^T, bf16 output (forward, dgrad).
 * Defined by "DeepGEMM Essentials", Parts 1 and 6 (LHS x RHS^T, LHS with
 * per-token 1x128 scales in the column-major layout of Part 5, RHS with
 * 128x128 block scales) and the reply in "[Help] Starter script for
 * nn.Linear for fwd,bwd" that the RHS scale row (1 x ceil(k/128)) of an
 * n-block serves every K block.  Within each 128-wide K block the products
 * are summed in fp32; each block's partial sum is multiplied by
 * sa(i, kb) * sb(j/128, kb) and added to an fp32 accumulator; the result is
 * rounded to bf16 (nearest, ties to even).
 *
 * A       E4M3 [m, k] row-major, k <= lda < 2^24, lda a multiple of 16; 16-B aligned.
 * sa      per-token scales in MN-major layout: sa_fmt FGFP8_SF_FP32 or
 *         FGFP8_SF_UE8M0: float (i, kb) at sa[kb*sa_ld + i];
 *         FGFP8_SF_PACKED_UE8M0: int32 word (i, kb/4) at sa[(kb/4)*sa_ld + i],
 *         exponent byte kb%4.  sa_ld >= m.
 * B       E4M3 [n, k] row-major, k <= ldb < 2^24, ldb a multiple of 16; 16-B aligned.
 * sb      fp32 [ceil(n/128), k/128] row-major: (nb, kb) at sb[nb*sb_ld + kb],
 *         sb_ld >= k/128.
 * D       bf16 [m, n] row-major, ldd >= n, multiple of 8; 16-B aligned.
 * k must be a positive multiple of 128; m, n >= 0 within the GEMM size limits
 * (FGFP8_MAX_GEMM_TILES, FGFP8_MAX_GEMM_N).
 */
int gemm_fp8_nt_bf16(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt, int64_t sa_ld,
                     const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld,
                     uint16_t *D, int64_t ldd, int64_t m, int64_t n, int64_t k,
                     void *stream);

/*
 * gemm_fp8_nt_bf16_splitk -- the same product as gemm_fp8_nt_bf16 (same
 * definition, passages and operand layouts) with K split over workgroups, for
 * products with too few output tiles to fill the GPU ("DeepGEMM Essentials",
 * Part 14: decode-sized products are bound by reading B once, so the work is
 * spread evenly over the compute units).
 *   m <= 64: the K blocks of all 128-column tiles are dealt out in equal
 *     consecutive shares, one per workgroup; a tile that a share covers whole
 *     is rounded and stored at once, and a tile split between shares gets the
 *     fp32 promoted partial sums of its shares added in share order by a
 *     second kernel, then rounded to bf16.
 *   m > 64: with at most 128 output tiles of 128x128, each tile's K blocks
 *     are cut into S consecutive slices, one workgroup per slice, and a second
 *     kernel adds each tile's S fp32 partial sums in slice order and rounds to
 *     bf16.  S is the largest of 2..4 with at least 8 K blocks per slice, and
 *     at least 12 when tiles * S exceeds 256.  With more tiles, or when no
 *     S >= 2 qualifies, the call runs gemm_fp8_nt_bf16's kernels and needs no
 *     workspace.
 * Deterministic: the same inputs give the same bits on every call.  Each
 * share's or slice's sum follows the definition above block by block; only
 * the grouping of the fp32 additions over K blocks differs from
 * gemm_fp8_nt_bf16, so the two agree to fp32 rounding, not bit for bit.
 *
 * workspace        device memory, 16-byte aligned, at least
 *                  gemm_fp8_nt_bf16_splitk_workspace(m, n, k) bytes, owned by
 *                  the caller; its contents on entry do not matter and are
 *                  overwritten.  May be NULL when that size is 0.  Calls that
 *                  share a workspace must be ordered (one stream, or events):
 *                  two in flight at once race.
 * Other arguments, errors, m, k, n and size limits as gemm_fp8_nt_bf16; also,
 * for m <= 64, FGFP8_EINVAL when ceil(n/128) * k/128 exceeds 2^31 - 16.
 */
int gemm_fp8_nt_bf16_splitk(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt, int64_t sa_ld,
                            const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld,
                            uint16_t *D, int64_t ldd, int64_t m, int64_t n, int64_t k,
                            void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gemm_fp8_nt_bf16_splitk_workspace -- bytes of workspace that
 * gemm_fp8_nt_bf16_splitk needs for (m, n, k).  m <= 64:
 * 2 * G * 16*ceil(m/16) * 128 * 4 (two partial-sum slots per workgroup), G the
 * number of workgroups (which depends on n and k only).  m > 64:
 * ceil(m/128) * ceil(n/128) * S * 128 * 128 * 4 (one slot per tile and K
 * slice, at most 32 MiB), or 0 when the plain kernels run.  0 when m or n is 0; FGFP8_EINVAL (-1) when m < 0,
 * n < 0, k is not a positive multiple of 128, or the size limits of
 * gemm_fp8_nt_bf16_splitk are exceeded.  Host only: launches
 * nothing and needs no device.
 */
int64_t gemm_fp8_nt_bf16_splitk_workspace(int64_t m, int64_t n, int64_t k);

/*
 * gemm_fp8_nt_bf16_splitk_noalloc -- gemm_fp8_nt_bf16_splitk without a
 * workspace argument, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The partial sums go to a static device array of the library
 * (FGFP8_SCRATCH_BYTES = 32 MiB per GPU, present from the library's load until
 * the process ends); the call itself allocates nothing.  Same kernels and
 * result bits as gemm_fp8_nt_bf16_splitk with a workspace.
 *
 * Limit: gemm_fp8_nt_bf16_splitk_workspace(m, n, k) must not exceed
 * FGFP8_SCRATCH_BYTES (for m = 64 up to about 3600 units of 128 columns x 128
 * K, e.g. n = k = 7168; for m > 64 up to 512 tile slices, which every plan
 * keeps to), else FGFP8_ESCRATCH and nothing is written.
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (two streams, or two threads) race and give wrong results, so order them.
 * Nothing in the array has to start at any value: each call writes every
 * partial sum before it reads it.
 * Arguments, layouts and the other errors as gemm_fp8_nt_bf16_splitk.
 */
int gemm_fp8_nt_bf16_splitk_noalloc(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt, int64_t sa_ld,
                                    const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld,
                                    uint16_t *D, int64_t ldd, int64_t m, int64_t n, int64_t k, void *stream);

/*
 * gemm_fp8_nt_bf16_cast -- gemm_fp8_nt_bf16 with the per-token FP8 cast of its
 * output fused into the epilogue, so that the next layer's FP8 operand leaves
 * the GEMM directly ("[Help] Starter script for nn.Linear for fwd,bwd": the
 * maintainers' advice to fuse as much as possible; the cast is "DeepGEMM
 * Essentials", Part 3, with 1 x 128 groups along n).
 *
 * A, sa, sa_fmt, sa_ld, B, ldb, sb, sb_ld, m, n, k   as gemm_fp8_nt_bf16.
 * D, ldd      the bf16 output as gemm_fp8_nt_bf16, or D == NULL to store only
 *             the FP8 output.
 * q, q_ld     E4M3 [m, n]: q_ld >= n, multiple of 4; q 4-byte aligned.
 * q_sf        fp32 scale of row i, 128-column group g at
 *             q_sf[i*q_sf_stride_row + g*q_sf_stride_group], g < ceil(n/128);
 *             row-major or MN-major as for cast_per_token.
 * q_sf_fmt    FGFP8_SF_FP32 or FGFP8_SF_UE8M0.
 * (q, q_sf) are bit-identical to cast_per_token(D, gran_k = 128, q_sf_fmt)
 * applied to the bf16 output D of the same call.
 */
int gemm_fp8_nt_bf16_cast(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt, int64_t sa_ld,
                          const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld,
                          uint16_t *D, int64_t ldd,
                          int q_sf_fmt, uint8_t *q, int64_t q_ld,
                          float *q_sf, int64_t q_sf_stride_row, int64_t q_sf_stride_group,
                          int64_t m, int64_t n, int64_t k, void *stream);

/*
 * gemm_fp8_nt_bf16_ue8m0_g32 -- D = (A * sa)(B * sb)^T with one power-of-two
 * scale per row and 32-wide K group on BOTH operands (the UE8M0 group-32
 * recipe that "deep-gemm: fused per-token FP8 cast in Triton" benchmarks):
 *     D[i, j] = sum_g 2^(ea(i,g) + eb(j,g)) sum_{t in g} A[i, t] B[j, t],
 * rounded to bf16 (nearest, ties to even).  Both operands are what
 * cast_per_token produces with gran_k = 32 and FGFP8_SF_PACKED_UE8M0 scales in
 * the MN-major layout.  The scales are applied by the gfx950 scaled FP8 MFMA,
 * which accumulates in fp32 across all of K.
 *
 * A    E4M3 [m, k] row-major, k <= lda < 2^24, lda a multiple of 16; 16-B aligned.
 * sa   int32 words, (i, kb) at sa[kb*sa_ld + i], sa_ld >= m: byte b of word
 *      (i, kb) is ea(i, 4kb + b) + 127.
 * B    E4M3 [n, k], as A.
 * sb   int32 words, (j, kb) at sb[kb*sb_ld + j], sb_ld >= n.
 * D    bf16 [m, n] row-major, ldd >= n, multiple of 8; 16-B aligned.
 * k must be a positive multiple of 128.  Products with 256 to 512 output tiles
 * of 256x256 (and k >= 1024) run a 256x256-tile kernel, the others 128x128
 * tiles; both give the same result.
 */
int gemm_fp8_nt_bf16_ue8m0_g32(const uint8_t *A, int64_t lda, const uint32_t *sa, int64_t sa_ld,
                               const uint8_t *B, int64_t ldb, const uint32_t *sb, int64_t sb_ld,
                               uint16_t *D, int64_t ldd, int64_t m, int64_t n, int64_t k,
                               void *stream);

/*
 * gemm_fp8_nt_bf16_ue8m0 -- gemm_fp8_nt_bf16 when every scale is a power of
 * two: A's 1x128 per-token scales and B's 128x128 block scales both come from
 * the casts' UE8M0 option ("deep-gemm: fused per-token FP8 cast in Triton";
 * the GEMM of "DeepGEMM Essentials", Parts 1 and 6):
 *     D[i, j] = sum_kb 2^(ea(i,kb) + eb(j/128,kb)) sum_{t in kb} A[i, t] B[j, t],
 * rounded to bf16.  The exponents are applied by the scaled FP8 MFMA, which
 * accumulates across K in fp32: no per-block promotion.  Products with 256 to
 * 512 output tiles of 256x256 (and k >= 1024) run a 256x256-tile kernel, the
 * others 128x128 tiles; both give the same result.
 *
 * sa_fmt   FGFP8_SF_UE8M0 (sa fp32 2^e, (i, kb) at sa[kb*sa_ld + i]) or
 *          FGFP8_SF_PACKED_UE8M0 (int32 words, byte kb%4 of word (i, kb/4) at
 *          sa[(kb/4)*sa_ld + i] is ea(i, kb) + 127).
 * sb       fp32 2^e [ceil(n/128), k/128], (nb, kb) at sb[nb*sb_ld + kb], as
 *          cast_per_block writes with FGFP8_SF_UE8M0.
 * A, lda, sa_ld, B, ldb, sb_ld, D, ldd, m, n, k   as gemm_fp8_nt_bf16.
 */
int gemm_fp8_nt_bf16_ue8m0(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt, int64_t sa_ld,
                           const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld,
                           uint16_t *D, int64_t ldd, int64_t m, int64_t n, int64_t k, void *stream);

/*
 * wgrad_gemm_fp8_nt_fp32_ue8m0 -- wgrad_gemm_fp8_nt_fp32 for operands whose
 * 1x128 per-token scales are powers of two on both sides (the UE8M0 option of
 * the per-token cast: "deep-gemm: fused per-token FP8 cast in Triton"; the
 * weight gradient of "DeepGEMM Essentials", Parts 12-13):
 *     D[i, j] += sum_kb 2^(ea(i,kb) + eb(j,kb)) sum_{t in kb} A[i, t] B[j, t].
 * The result equals wgrad_gemm_fp8_nt_fp32 on the same scales as fp32 values
 * up to rounding order: the exponents are applied by the scaled FP8 MFMA,
 * which accumulates across K in fp32, so no per-block promotion is needed.
 *
 * sf_fmt   FGFP8_SF_UE8M0: sa, sb are fp32 2^e values, (i, kb) at
 *          sa[kb*sa_ld + i] and (j, kb) at sb[kb*sb_ld + j] (what
 *          cast_per_token writes with gran_k = 128 into MN-major views);
 *          FGFP8_SF_PACKED_UE8M0: int32 words, byte kb%4 of word
 *          (i, kb/4) at sa[(kb/4)*sa_ld + i] is ea(i, kb) + 127 (likewise sb).
 * A, lda, sa_ld, B, ldb, sb_ld, D, ldd, m, n, k   as wgrad_gemm_fp8_nt_fp32
 *          (sa_ld >= m, sb_ld >= n).
 */
int wgrad_gemm_fp8_nt_fp32_ue8m0(const uint8_t *A, int64_t lda, const void *sa, int sf_fmt, int64_t sa_ld,
                                 const uint8_t *B, int64_t ldb, const void *sb, int64_t sb_ld,
                                 float *D, int64_t ldd, int64_t m, int64_t n, int64_t k, void *stream);

/*
 * wgrad_gemm_fp8_nt_fp32_ue8m0_g32 -- the weight-gradient form of the UE8M0
 * group-32 recipe: D += (A * sa)(B * sb)^T in fp32, with K running over tokens
 * ("DeepGEMM Essentials", Parts 12-13: dW = dY^T x, fp32 output accumulated in
 * place), and one power-of-two scale per row and 32-wide K group on both
 * operands, applied by the scaled FP8 MFMA:
 *     D[i, j] += sum_g 2^(ea(i,g) + eb(j,g)) sum_{t in g} A[i, t] B[j, t].
 * Both operands are what cast_per_token produces from the transposed views
 * (dY^T, x^T) with gran_k = 32 and FGFP8_SF_PACKED_UE8M0 scales, MN-major.
 *
 * A, sa, sa_ld, B, sb, sb_ld, m, n, k   as gemm_fp8_nt_bf16_ue8m0_g32.
 * D    fp32 [m, n] row-major, read and written; ldd >= n, multiple of 4;
 *      16-B aligned.
 */
int wgrad_gemm_fp8_nt_fp32_ue8m0_g32(const uint8_t *A, int64_t lda, const uint32_t *sa, int64_t sa_ld,
                                     const uint8_t *B, int64_t ldb, const uint32_t *sb, int64_t sb_ld,
                                     float *D, int64_t ldd, int64_t m, int64_t n, int64_t k,
                                     void *stream);

/*
 * m_grouped_gemm_fp8_nt_bf16_contiguous -- the forward GEMM of a mixture of
 * experts over a token-contiguous LHS.  Defined by "DeepGEMM Essentials",
 * Parts 8-11: the tokens routed to expert e are consecutive rows of A, each
 * expert's run of rows is padded to a multiple of 128 (the contiguous-layout
 * alignment), and m_indices[i] is the expert of row i, or -1 for a padding
 * row.  Row i with m_indices[i] = e >= 0 gets
 *     D[i, :] = (A[i] * sa[i]) (B_e * sb_e)^T,
 * computed exactly as gemm_fp8_nt_bf16 computes a row; padding rows of D are
 * not written.
 *
 * A, sa, sa_fmt, sa_ld, D, ldd, m, n, k   as gemm_fp8_nt_bf16 (m = all rows,
 *          padding included).
 * B        expert e's E4M3 [n, k] weights at B + e*b_expert_stride (bytes),
 *          row-major with ldb; b_expert_stride >= (n-1)*ldb + k and a multiple
 *          of 16.
 * sb       expert e's fp32 [ceil(n/128), k/128] block scales at
 *          sb + e*sb_expert_stride (floats), (nb, kb) at nb*sb_ld + kb.
 * m_indices int32 [m], device memory; num_experts >= 1.
 * Layout requirement (the contiguous layout above): every 128-row block
 * [128t, 128t+128) of A holds rows of one expert and padding only.  A block
 * is computed for the largest id among its rows; rows of any other expert in
 * the block, rows with -1, and blocks whose id is not in [0, num_experts)
 * are left unwritten (no memory outside the experts' weights is read).
 */
int m_grouped_gemm_fp8_nt_bf16_contiguous(const uint8_t *A, int64_t lda, const void *sa, int sa_fmt,
                                          int64_t sa_ld, const uint8_t *B, int64_t ldb,
                                          int64_t b_expert_stride, const float *sb, int64_t sb_ld,
                                          int64_t sb_expert_stride, const int32_t *m_indices,
                                          int64_t num_experts, uint16_t *D, int64_t ldd, int64_t m,
                                          int64_t n, int64_t k, void *stream);

/*
 * m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous -- the m-grouped contiguous
 * GEMM of m_grouped_gemm_fp8_nt_bf16_contiguous in the UE8M0 group-32 recipe
 * (the packed-UE8M0 group-32 scales that "deep-gemm: fused per-token FP8 cast
 * in Triton" names for MoE): row i with m_indices[i] = e >= 0 gets
 *     D[i, :] = (A[i] * sa[i]) (B_e * sb_e)^T,
 * computed exactly as gemm_fp8_nt_bf16_ue8m0_g32 computes a row.
 *
 * A, sa, sa_ld, D, ldd, m, n, k   as gemm_fp8_nt_bf16_ue8m0_g32 (m = all rows,
 *          padding included).
 * B        expert e's E4M3 [n, k] at B + e*b_expert_stride (bytes), as in
 *          m_grouped_gemm_fp8_nt_bf16_contiguous.
 * sb       expert e's packed words at sb + e*sb_expert_stride (int32 words),
 *          (j, kb) at [kb*sb_ld + j], sb_ld >= n; sb_expert_stride >=
 *          (k/128 - 1)*sb_ld + n.
 * m_indices, num_experts and the layout requirement as in
 *          m_grouped_gemm_fp8_nt_bf16_contiguous.
 */
int m_grouped_gemm_fp8_nt_bf16_ue8m0_g32_contiguous(const uint8_t *A, int64_t lda, const uint32_t *sa,
                                                    int64_t sa_ld, const uint8_t *B, int64_t ldb,
                                                    int64_t b_expert_stride, const uint32_t *sb, int64_t sb_ld,
                                                    int64_t sb_expert_stride, const int32_t *m_indices,
                                                    int64_t num_experts, uint16_t *D, int64_t ldd, int64_t m,
                                                    int64_t n, int64_t k, void *stream);

/*
 * wgrad_gemm_fp8_nt_fp32 -- D += (A * sa)(B * sb)^T in fp32 (weight gradient).
 * Defined by "DeepGEMM Essentials", Parts 12-13 (the weight gradient is
 * accumulated into an existing fp32 tensor, expected = original + dY^T x)
 * and the wgrad line of the pseudo-code in "[Help] Starter script for
 * nn.Linear for fwd,bwd" (both operands transposed so that K runs over
 * tokens).  Both operands carry one scale per row and 128-wide K block; each
 * K block's fp32 partial sum is multiplied by sa(i, kb) * sb(j, kb).
 *
 * A   E4M3 [m, k] (m = output features, k = tokens), k <= lda < 2^24, multiple of 16.
 * sa  fp32 (i, kb) at sa[kb*sa_ld + i], sa_ld >= m.
 * B   E4M3 [n, k] (n = input features), k <= ldb < 2^24, multiple of 16.
 * sb  fp32 (j, kb) at sb[kb*sb_ld + j], sb_ld >= n.
 * D   fp32 [m, n] row-major, ldd >= n, multiple of 4; read and written.
 * k must be a positive multiple of 128.
 */
int wgrad_gemm_fp8_nt_fp32(const uint8_t *A, int64_t lda, const float *sa, int64_t sa_ld,
                           const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_ld,
                           float *D, int64_t ldd, int64_t m, int64_t n, int64_t k,
                           void *stream);

/* Human-readable text of a return code (static storage). */
const char *fgfp8_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FGFP8_H */
