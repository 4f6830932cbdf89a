/*
 * fgfp8_oracle.c -- CPU oracle for the fine-grained block-scaled FP8 path.
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  This is a plain, slow, obviously
 * correct CPU implementation of what the GPU library computes.  Only the
 * tests, the smoke check and the benchmark's CPU-baseline leg may load it.
 * It shares no code, header, table or constant generator with the HIP
 * library, and neither side includes the other.
 *
 * Sources (web pages; cited by title and section):
 *   [P1] "[Help] Starter script for nn.Linear for fwd,bwd" (DeepGEMM issue
 *        #102): the maintainer's forward / dgrad / wgrad pseudo-code, and the
 *        reply explaining that each n-block reads one whole row
 *        (1 x ceil(k/128)) of the RHS 128x128 scale grid for all K blocks.
 *   [P2] "DeepGEMM Essentials: High-Performance FP8 Matrix Multiplication"
 *        (dev.to): Part 3 (per-token cast), Part 4 (128x128 block cast),
 *        Part 5 (column-major LHS scales), Part 6 (the NT GEMM call),
 *        Parts 12-13 (wgrad accumulates into an fp32 tensor).
 *   [P3] "deep-gemm: fused per-token FP8 cast in Triton" (kernels-community
 *        PR #1326): use_ue8m0 / gran_k / packed-UE8M0 options, bf16 or fp32
 *        input, and the correctly rounded reciprocal.
 *
 * Readings taken where the pages leave a step open (each is listed in the
 * design notes):
 *   - fp32-scale multiplier is 448/amax as PyTorch evaluates it for a scalar
 *     over a tensor: fl(fl(1/amax) * 448) ([P2] Part 3 code; [P3] "div_rn").
 *   - UE8M0 scale is the next power of two at or above fl(amax/448), found
 *     from the fp32 bits; the multiplier is its exact reciprocal.
 *   - packed UE8M0: byte (e + 127); group 4w+b sits in byte b of int32 word w;
 *     unused bytes of the last word are zero.
 *   - a partial last group / block takes its amax over valid elements only
 *     (the zero padding of [P2] Parts 3-4 cannot raise an amax).
 *   - GEMM partial sums are exact per 128-wide K block in fp64, scaled by
 *     sa*sb and summed in fp64.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * Every fp32 operation below is a single IEEE-754 binary32 operation rounded
 * to nearest even (x86-64 SSE arithmetic, no contraction into FMA).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Input dtypes and scale formats (argument meaning as in the library). */
enum { ORC_IN_BF16 = 0, ORC_IN_FP32 = 1 };
enum { ORC_SF_FP32 = 0, ORC_SF_UE8M0 = 1, ORC_SF_PACKED_UE8M0 = 2 };

static uint32_t f32_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }
static float f32_from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }

/* ------------------------------------------------------------------------
 * OCP FP8 E4M3 ("fn" variant): sign, 4-bit exponent with bias 7, 3-bit
 * mantissa.  No infinities; S.1111.111 is NaN; largest finite value is
 * 1.75 * 2^8 = 448; subnormals are m * 2^-9 for m = 1..7.
 * ---------------------------------------------------------------------- */

/* Exact value of an E4M3 code (NaN for the two NaN codes). */
static double e4m3_value(uint8_t code)
{
    int neg = code >> 7, ex = (code >> 3) & 15, man = code & 7;
    double mag;
    if (ex == 15 && man == 7) return NAN;
    if (ex == 0) mag = ldexp((double)man, -9);          /* subnormal */
    else mag = ldexp((double)(8 + man), ex - 10);       /* (1 + man/8) * 2^(ex-7) */
    return neg ? -mag : mag;
}

/* Round an fp32 value to E4M3, nearest with ties to even mantissa, in the
 * normal and subnormal ranges alike.  A result above 448 has no finite
 * encoding and becomes NaN (no saturation); the sign is kept, so -0 -> 0x80. */
static uint8_t e4m3_round(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a, quantum, n, r;
    int e2, top;
    if (isnan(v) || isinf(v)) return sign | 0x7f;
    a = fabs((double)v);
    if (a == 0.0) return sign;
    frexp(a, &e2);
    top = e2 - 1;                       /* a lies in [2^top, 2^(top+1)) */
    if (top < -6) top = -6;             /* subnormals share the quantum of the lowest binade */
    quantum = ldexp(1.0, top - 3);      /* 3 mantissa bits */
    n = nearbyint(a / quantum);         /* a/quantum is exact; default mode rounds ties to even */
    r = n * quantum;                    /* exact */
    if (r > 448.0) return sign | 0x7f;
    if (r < ldexp(1.0, -6)) return sign | (uint8_t)(r / ldexp(1.0, -9));
    frexp(r, &e2);
    top = e2 - 1;
    return sign | (uint8_t)((top + 7) << 3) | (uint8_t)(r / ldexp(1.0, top - 3) - 8.0);
}

/* ------------------------------------------------------------------------
 * Per-group scale ([P2] Part 3; formats from [P3]).
 * ---------------------------------------------------------------------- */
typedef struct {
    float sf;    /* scale written out (fp32 bits, or 2^e for UE8M0) */
    float mult;  /* multiplier applied to every element of the group */
    int e;       /* UE8M0 exponent (unused for fp32 scales) */
} group_scale;

static group_scale scale_from_amax(float amax, int sf_fmt)
{
    const float amax_floor = 1e-4f;     /* clamp(1e-4) on an fp32 tensor uses fp32(1e-4) */
    group_scale g;
    float s;
    if (amax < amax_floor) amax = amax_floor;
    s = amax / 448.0f;                  /* dequantisation scale, correctly rounded */
    if (sf_fmt == ORC_SF_FP32) {
        float recip = 1.0f / amax;      /* correctly rounded reciprocal ... */
        g.sf = s;
        g.mult = recip * 448.0f;        /* ... then times 448: two roundings */
        g.e = 0;
    } else {
        uint32_t b = f32_bits(s);
        int biased = (int)((b >> 23) & 0xff);
        int e = biased - 127 + ((b & 0x7fffff) != 0);   /* smallest e with 2^e >= s */
        g.e = e;
        g.sf = f32_from_bits((uint32_t)(e + 127) << 23);
        g.mult = f32_from_bits((uint32_t)(127 - e) << 23);
    }
    return g;
}

static float load_x(const void *x, int dtype, int64_t off)
{
    if (dtype == ORC_IN_BF16) {
        uint16_t h = ((const uint16_t *)x)[off];
        return f32_from_bits((uint32_t)h << 16);        /* bf16 widens exactly */
    }
    return ((const float *)x)[off];
}

/* ------------------------------------------------------------------------
 * Per-token cast: every row, every 1 x gran group along the columns.
 * x(r, c) = x[r*xs_row + c*xs_col]; q(r, c) = q[r*q_ld + c].
 * fp32 / UE8M0: scale (r, g) at ((float*)sf)[r*sf_s_row + g*sf_s_grp].
 * packed:        word  (r, w) at ((int32*)sf)[r*sf_s_row + w*sf_s_grp].
 * ---------------------------------------------------------------------- */
int orc_cast_per_token(const void *x, int x_dtype, int64_t rows, int64_t cols,
                       int64_t xs_row, int64_t xs_col, int gran, int sf_fmt,
                       uint8_t *q, int64_t q_ld, void *sf, int64_t sf_s_row, int64_t sf_s_grp)
{
    int64_t groups, r;
    if (gran != 32 && gran != 128) return -1;
    if (x_dtype != ORC_IN_BF16 && x_dtype != ORC_IN_FP32) return -1;
    if (sf_fmt < ORC_SF_FP32 || sf_fmt > ORC_SF_PACKED_UE8M0) return -1;
    if (rows <= 0 || cols <= 0) return 0;
    groups = (cols + gran - 1) / gran;

#pragma omp parallel for schedule(static)
    for (r = 0; r < rows; ++r) {
        int64_t g, c;
        uint32_t word = 0;                  /* packed mode: exponent bytes of groups 4w..4w+3 */
        for (g = 0; g < groups; ++g) {
            int64_t c0 = g * gran, c1 = c0 + gran < cols ? c0 + gran : cols;
            float amax = 0.0f;
            group_scale s;
            /* step 1: amax over the valid elements of the group */
            for (c = c0; c < c1; ++c) {
                float a = fabsf(load_x(x, x_dtype, r * xs_row + c * xs_col));
                if (a > amax) amax = a;
            }
            /* steps 2-3: clamp, scale and multiplier */
            s = scale_from_amax(amax, sf_fmt);
            /* step 4: quantise */
            for (c = c0; c < c1; ++c) {
                float v = load_x(x, x_dtype, r * xs_row + c * xs_col) * s.mult;
                q[r * q_ld + c] = e4m3_round(v);
            }
            /* step 5: scale store */
            if (sf_fmt != ORC_SF_PACKED_UE8M0) {
                ((float *)sf)[r * sf_s_row + g * sf_s_grp] = s.sf;
            } else {
                word |= (uint32_t)(s.e + 127) << (8 * (g % 4));
                if (g % 4 == 3 || g == groups - 1) {
                    ((uint32_t *)sf)[r * sf_s_row + (g / 4) * sf_s_grp] = word;
                    word = 0;
                }
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Per-block cast ([P2] Part 4): 128 x 128 blocks over a row-major matrix.
 * Scale of block (bi, bj) at sf[bi*sf_ld + bj]; fp32 or UE8M0 only.
 * ---------------------------------------------------------------------- */
int orc_cast_per_block(const void *x, int x_dtype, int64_t rows, int64_t cols, int64_t x_ld,
                       int sf_fmt, uint8_t *q, int64_t q_ld, float *sf, int64_t sf_ld)
{
    int64_t brows, bcols, blk;
    if (x_dtype != ORC_IN_BF16 && x_dtype != ORC_IN_FP32) return -1;
    if (sf_fmt != ORC_SF_FP32 && sf_fmt != ORC_SF_UE8M0) return -1;
    if (rows <= 0 || cols <= 0) return 0;
    brows = (rows + 127) / 128;
    bcols = (cols + 127) / 128;

#pragma omp parallel for schedule(static)
    for (blk = 0; blk < brows * bcols; ++blk) {
        int64_t bi = blk / bcols, bj = blk % bcols, r, c;
        int64_t r0 = bi * 128, r1 = r0 + 128 < rows ? r0 + 128 : rows;
        int64_t c0 = bj * 128, c1 = c0 + 128 < cols ? c0 + 128 : cols;
        float amax = 0.0f;
        group_scale s;
        for (r = r0; r < r1; ++r)
            for (c = c0; c < c1; ++c) {
                float a = fabsf(load_x(x, x_dtype, r * x_ld + c));
                if (a > amax) amax = a;
            }
        s = scale_from_amax(amax, sf_fmt);
        for (r = r0; r < r1; ++r)
            for (c = c0; c < c1; ++c)
                q[r * q_ld + c] = e4m3_round(load_x(x, x_dtype, r * x_ld + c) * s.mult);
        sf[bi * sf_ld + bj] = s.sf;
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Block-scaled NT GEMM reference ([P2] Parts 1, 6, 13; [P1]).
 *   ref(i, j) = sum_kb  P(i, j, kb) * sa(i, kb) * sb(j', kb)
 *   P(i, j, kb) = sum_{t < 128} A(i, 128kb + t) * B(j, 128kb + t)
 * A(i, t) = dec(A[i*lda + t]),  B(j, t) = dec(B[j*ldb + t]).
 * sa(i, kb) = sa[i*sa_si + kb*sa_sk].
 * sb: block mode (sb_rows_per_scale = 128) uses j' = j / 128 (one scale per
 * 128 x 128 block); row mode (sb_rows_per_scale = 1) uses j' = j.
 * sb(j', kb) = sb[j'*sb_sj + kb*sb_sk].
 * P is exact in fp64: each product of two E4M3 values has at most 8
 * significant bits and lies in [2^-18, 2^17], so 128 of them sum exactly
 * within 53 bits.  absum(i, j) = sum_kb |sa*sb| * sum_t |A*B| bounds the
 * rounding an fp32 accumulation may add.
 * When idx_i / idx_j are given, only those `count` outputs are computed,
 * otherwise all m*n in row-major order (count ignored).
 * ---------------------------------------------------------------------- */
int orc_gemm_nt(const uint8_t *A, int64_t lda, const float *sa, int64_t sa_si, int64_t sa_sk,
                const uint8_t *B, int64_t ldb, const float *sb, int64_t sb_sj, int64_t sb_sk,
                int sb_rows_per_scale, int64_t m, int64_t n, int64_t k,
                const int64_t *idx_i, const int64_t *idx_j, int64_t count,
                double *ref, double *absum)
{
    double lut[256];
    int64_t total, o, kblocks;
    int c;
    if (k % 128 != 0) return -1;
    if (sb_rows_per_scale != 1 && sb_rows_per_scale != 128) return -1;
    for (c = 0; c < 256; ++c) lut[c] = e4m3_value((uint8_t)c);
    kblocks = k / 128;
    total = (idx_i && idx_j) ? count : m * n;

#pragma omp parallel for schedule(dynamic, 64)
    for (o = 0; o < total; ++o) {
        int64_t i = (idx_i && idx_j) ? idx_i[o] : o / n;
        int64_t j = (idx_i && idx_j) ? idx_j[o] : o % n;
        int64_t jb = j / sb_rows_per_scale, kb, t;
        double acc = 0.0, mag = 0.0;
        for (kb = 0; kb < kblocks; ++kb) {
            double p = 0.0, pabs = 0.0, s;
            for (t = 128 * kb; t < 128 * kb + 128; ++t) {
                double prod = lut[A[i * lda + t]] * lut[B[j * ldb + t]];
                p += prod;
                pabs += fabs(prod);
            }
            s = (double)sa[i * sa_si + kb * sa_sk] * (double)sb[jb * sb_sj + kb * sb_sk];
            acc += p * s;
            mag += pabs * fabs(s);
        }
        ref[o] = acc;
        if (absum) absum[o] = mag;
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Small helpers the tests use.
 * ---------------------------------------------------------------------- */

/* fp32 -> E4M3 codes, element-wise. */
void orc_e4m3_round_array(const float *v, int64_t n, uint8_t *out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = e4m3_round(v[i]);
}

/* E4M3 codes -> exact values. */
void orc_e4m3_value_array(const uint8_t *codes, int64_t n, double *out)
{
    int64_t i;
    for (i = 0; i < n; ++i) out[i] = e4m3_value(codes[i]);
}

/* fp64 -> bf16 bits, nearest with ties to even, rounded once from fp64. */
void orc_round_bf16_array(const double *v, int64_t n, uint16_t *out)
{
    int64_t i;
    for (i = 0; i < n; ++i) {
        double a = fabs(v[i]), quantum, r;
        int e2;
        uint8_t neg = signbit(v[i]) ? 1 : 0;
        uint32_t b;
        if (a == 0.0 || isnan(v[i])) {
            out[i] = isnan(v[i]) ? 0x7fc0 : (uint16_t)(neg << 15);
            continue;
        }
        frexp(a, &e2);
        if (e2 - 1 < -126) e2 = -125;                   /* subnormal quantum 2^-133 */
        quantum = ldexp(1.0, e2 - 1 - 7);               /* 8 significant bits */
        r = nearbyint(a / quantum) * quantum;           /* may carry into the next binade */
        if (r >= ldexp(1.0, 128)) b = 0x7f800000u;       /* overflow to infinity */
        else b = f32_bits((float)r);                     /* exact: r has <= 8 significant bits */
        out[i] = (uint16_t)((b >> 16) | (neg << 15));
    }
}

void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
