// cast.hip -- per-token and per-block FP8 (E4M3) cast kernels for gfx950.
//
// The cast is defined in "DeepGEMM Essentials: High-Performance FP8 Matrix
// Multiplication", Part 3 (per token: amax of each 1x128 group along a row,
// clamped at 1e-4; scale amax/448; each element times 448/amax rounded to
// E4M3) and Part 4 (the same over 128x128 blocks), with the group-32,
// UE8M0 and packed-UE8M0 options of "deep-gemm: fused per-token FP8 cast in
// Triton".  Each kernel is one pass over HBM: every input byte is read once,
// every output byte written once.
#include "device_common.h"
#include "launch.h"

#pragma clang fp contract(off)

namespace fgfp8 {
namespace {

constexpr int kThreads = 256;

template <typename T>
__device__ __forceinline__ void load8(const T *p, bool full, int valid, float (&v)[8]);

// 8 bf16 (16 bytes) -> fp32; partial chunks read element by element.
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, bool full, int valid, float (&v)[8]) {
  if (full) {
    const uint4 w = *reinterpret_cast<const uint4 *>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < valid ? __uint_as_float((uint32_t)p[e] << 16) : 0.0f;
  }
}

// 8 fp32 (two 16-byte loads).
template <>
__device__ __forceinline__ void load8<float>(const float *p, bool full, int valid, float (&v)[8]) {
  if (full) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = e < valid ? p[e] : 0.0f;
  }
}

__device__ __forceinline__ uint32_t abs_bits(float f) { return __float_as_uint(f) & 0x7FFFFFFFu; }

// ---------------------------------------------------------------------------
// Per-token cast, row-major input.
//
// A "task" is one wave-wide step over a row: 64 lanes x 16 elements = 1024
// consecutive columns, i.e. 8 groups of 128 (8 lanes each) or 32 groups of 32
// (2 lanes each).  Each wave walks a contiguous range of tasks, U tasks at a
// time so that 2*U (bf16) or 4*U (fp32) 16-byte loads per lane are in flight;
// E4M3 bytes leave as one 16-byte store per lane.  The group amax is reduced
// with DPP inside the 16-lane rows; packed UE8M0 words are assembled with a
// DPP OR (group 32) or readlanes (group 128).
//
// Task order.  Row-major (QUAD = false): task t is step t % steps of row
// t / steps.  With MN-major scales (element (r, g) at g*ld + r) the U = 4 tasks
// of a batch are instead four consecutive rows at the same column step
// (QUAD = true), so the four scales of each group are contiguous and leave as
// one 16-byte store, not four scattered 4-byte ones.  Hardware workgroup b runs
// on XCD b % 8; the logical numbering puts eight consecutive workgroups (the
// 32 rows of a 128-byte line of MN-major scales) on one XCD, so the line is
// assembled in one L2 and reaches memory whole.  (Measured on MI355X: giving
// each XCD one contiguous band of rows instead is 14% slower for 16384 x 4096,
// whose bands then start 2^24 bytes apart.)
// ---------------------------------------------------------------------------
constexpr int kTokEl = 16;              // elements per lane per task
constexpr int kTokSpan = 64 * kTokEl;   // columns per task

// 16 elements kept as raw words until they are processed (8 words of bf16
// pairs, or 16 fp32 words), so that U tasks of loads stay in flight cheaply.
template <typename T>
struct Raw16 {
  static constexpr int kWords = 8 * (int)sizeof(T) / 2;
  uint32_t w[kWords];
  __device__ __forceinline__ float get(int e) const {
    if constexpr (sizeof(T) == 2) return (e & 1) ? bf16_hi(w[e >> 1]) : bf16_lo(w[e >> 1]);
    else return __uint_as_float(w[e]);
  }
};

template <typename T>
__device__ __forceinline__ void load16(const T *p, bool full, int valid, Raw16<T> &r) {
  if (full) {
#pragma unroll
    for (int i = 0; i < Raw16<T>::kWords / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4 *>(p)[i];
      r.w[4 * i] = v.x; r.w[4 * i + 1] = v.y; r.w[4 * i + 2] = v.z; r.w[4 * i + 3] = v.w;
    }
  } else if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = 2 * i < valid ? (uint32_t)p[2 * i] : 0u;
      const uint32_t hi = 2 * i + 1 < valid ? (uint32_t)p[2 * i + 1] : 0u;
      r.w[i] = lo | (hi << 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) r.w[i] = i < valid ? __float_as_uint(p[i]) : 0u;
  }
}

template <typename TIn, int GRAN, int FMT, bool Q16, bool QUAD>
__global__ __launch_bounds__(kThreads) void cast_tok_rows_kernel(
    const TIn *__restrict__ x, int64_t rows, int64_t cols, int64_t xs_row, uint8_t *__restrict__ q, int64_t q_ld,
    void *__restrict__ sf, int64_t sf_s_row, int64_t sf_s_grp, int64_t steps_per_row, int64_t tasks,
    int64_t tasks_per_wave) {
  constexpr int L = GRAN / kTokEl;  // lanes per group
  constexpr int U = 4;
  constexpr bool kUe8m0 = FMT != kSfFp32;
  const int lane = threadIdx.x & 63;
  // Within each run of 64 workgroups, logical workgroup 8i + x is hardware
  // workgroup 8x + i, which runs on XCD i: eight consecutive logical workgroups
  // share an XCD, and the XCDs still interleave at that grain.
  // (a grid of fewer than 64 workgroups keeps the hardware order)
  const int64_t b = blockIdx.x;
  const int64_t blk = gridDim.x < 64 ? b : (b & ~(int64_t)63) | ((b & 7) << 3) | ((b >> 3) & 7);
  const int64_t wave = blk * (kThreads / kWave) + (threadIdx.x >> 6);
  const int64_t t_begin = wave * tasks_per_wave;
  const int64_t t_end = min(t_begin + tasks_per_wave, tasks);

  for (int64_t tb = t_begin; tb < t_end; tb += U) {
    Raw16<TIn> raw[U];
    int64_t row[U], col[U];
    uint32_t sv[U];   // QUAD: the batch's scale (or packed word) per row, stored after the batch
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = tb + u;
      row[u] = 0;
      col[u] = cols;  // marks the lane idle
      sv[u] = 0u;
      if (t < t_end) {
        int64_t r, s;
        if constexpr (QUAD) {   // tasks 4i..4i+3 of row quad R: rows 4R..4R+3 at step i
          const int64_t quad = t / (4 * steps_per_row);
          const int64_t rem = t - quad * 4 * steps_per_row;
          s = rem >> 2;
          r = 4 * quad + (rem & 3);
        } else {
          r = t / steps_per_row;
          s = t - r * steps_per_row;
        }
        row[u] = r;
        if (r < rows) col[u] = s * kTokSpan + (int64_t)lane * kTokEl;
      }
      if (col[u] < cols) {
        load16<TIn>(x + row[u] * xs_row + col[u], col[u] + kTokEl <= cols, (int)min<int64_t>(cols - col[u], kTokEl), raw[u]);
      } else {
#pragma unroll
        for (int i = 0; i < Raw16<TIn>::kWords; ++i) raw[u].w[i] = 0u;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tb + u >= t_end) break;  // uniform across the wave
      float v[kTokEl];
#pragma unroll
      for (int e = 0; e < kTokEl; ++e) v[e] = raw[u].get(e);
      uint32_t am = 0;
#pragma unroll
      for (int e = 0; e < kTokEl; ++e) am = max(am, abs_bits(v[e]));
      am = group_max_u32<L>(am);
      const GroupScale gs = group_scale<kUe8m0>(__uint_as_float(am));
      const float mu = gs.mult;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = e4m3x4(v[4 * e] * mu, v[4 * e + 1] * mu, v[4 * e + 2] * mu, v[4 * e + 3] * mu);
      const int64_t c = col[u];
      uint8_t *qp = q + row[u] * q_ld + c;
      if (c + kTokEl <= cols) {
        if constexpr (Q16) {
          *reinterpret_cast<uint4 *>(qp) = make_uint4(w[0], w[1], w[2], w[3]);
        } else {
          reinterpret_cast<uint2 *>(qp)[0] = make_uint2(w[0], w[1]);
          reinterpret_cast<uint2 *>(qp)[1] = make_uint2(w[2], w[3]);
        }
      } else if (c < cols) {
        const int valid = (int)(cols - c);
#pragma unroll
        for (int e = 0; e < kTokEl; ++e)
          if (e < valid) qp[e] = (uint8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xFFu);
      }
      const int64_t g = c / GRAN;  // group of this lane
      if constexpr (FMT != kSfPackedUe8m0) {
        if constexpr (QUAD) sv[u] = __float_as_uint(gs.sf);
        else if ((lane % L) == 0 && c < cols)
          reinterpret_cast<float *>(sf)[row[u] * sf_s_row + g * sf_s_grp] = gs.sf;
      } else {
        const uint32_t mine = c < cols ? gs.e8 << (8 * (g & 3)) : 0u;
        uint32_t word;
        if constexpr (GRAN == 32) {
          word = group_or_u32<8>(mine);   // 4 groups x 2 lanes
        } else {
          const uint32_t r16 = group_or_u32<16>(mine);   // 2 groups x 8 lanes per 16-lane row
          const int base = lane & 32;                      // lanes 0-31 -> word 2s, 32-63 -> word 2s+1
          word = (uint32_t)__builtin_amdgcn_readlane((int)r16, 0) | (uint32_t)__builtin_amdgcn_readlane((int)r16, 16);
          const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)r16, 32) |
                              (uint32_t)__builtin_amdgcn_readlane((int)r16, 48);
          if (base) word = hi;
        }
        if constexpr (QUAD) sv[u] = word;
        else if ((lane % (4 * L)) == 0 && c < cols)
          reinterpret_cast<uint32_t *>(sf)[row[u] * sf_s_row + (g >> 2) * sf_s_grp] = word;
      }
    }
    if constexpr (QUAD) {
      // rows row[0] .. row[0]+3 (a multiple of 4; rows past the end were idle) at
      // the same column: MN-major scales (s_row == 1, s_grp % 4 == 0, 16-byte
      // aligned base) put the four values of a group side by side
      constexpr int W = FMT == kSfPackedUe8m0 ? 4 * L : L;   // lanes per stored unit
      const int64_t c = col[0], r0 = row[0];
      const int64_t unit = FMT == kSfPackedUe8m0 ? c / GRAN / 4 : c / GRAN;
      if ((lane % W) == 0 && c < cols) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(sf) + unit * sf_s_grp + r0;
        if (r0 + 4 <= rows) {
          *reinterpret_cast<uint4 *>(dst) = make_uint4(sv[0], sv[1], sv[2], sv[3]);
        } else {
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (r0 + u < rows) dst[u] = sv[u];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Per-token cast of a transposed view (the wgrad operands: groups run along
// the tokens, which are the rows of the underlying row-major matrix).
//
// One workgroup owns 64 features (rows of the view) x 128 tokens (columns of
// the view).  Phase 1 reads the tile with coalesced 16-byte loads along the
// features and writes it to LDS transposed (fp32); phase 2 lets each thread
// own 32 consecutive tokens of one feature, so the group amax needs at most a
// 4-lane DPP reduction and the E4M3 row is written with 16-byte stores.  The
// LDS column index is XOR-swizzled so both phases are free of bank conflicts.
// For packed UE8M0 with group 128 a word spans 512 tokens, so a workgroup
// then walks 4 tiles along the tokens.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int tile_col(int f, int tok) {
  const int s = (((tok >> 5) & 3) << 2) ^ (((f >> 3) & 3) << 3) ^ ((f & 1) << 4);
  return f * 128 + (tok ^ s);
}

template <typename TIn, int GRAN, int FMT>
__global__ __launch_bounds__(kThreads) void cast_tok_cols_kernel(
    const TIn *__restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint8_t *__restrict__ q,
    int64_t q_ld, void *__restrict__ sf, int64_t sf_s_row, int64_t sf_s_grp) {
  constexpr int NT = (FMT == kSfPackedUe8m0 && GRAN == 128) ? 4 : 1;
  constexpr bool kUe8m0 = FMT != kSfFp32;
  __shared__ __attribute__((aligned(16))) float tile[64 * 128];
  const int t = threadIdx.x;
  const int64_t f0 = (int64_t)blockIdx.x * 64;
  const int64_t cbase = (int64_t)blockIdx.y * (128 * NT);
  const int fl = t >> 2, p = t & 3;  // phase 2: feature, 32-token part
  const int64_t f = f0 + fl;
  uint32_t word128 = 0;

  for (int it = 0; it < NT; ++it) {
    const int64_t c0 = cbase + (int64_t)it * 128;
    if (c0 >= cols) break;  // uniform
    // ---- phase 1: global -> LDS (transposed) ----
    if constexpr (sizeof(TIn) == 2) {
      const int tr = t >> 3, fc = t & 7;
      const int64_t fb = f0 + 8 * fc;
      const bool fullf = fb + 8 <= rows;
      const int validf = (int)max<int64_t>(0, min<int64_t>(8, rows - fb));
      float v[4][8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t c = c0 + 32 * i + tr;
        if (c < cols && validf > 0) {
          load8<TIn>(x + c * ld + fb, fullf, validf, v[i]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) tile[tile_col(8 * fc + e, 32 * i + tr)] = v[i][e];
    } else {
      const int tr = t >> 4, fc = t & 15;
      const int64_t fb = f0 + 4 * fc;
      const bool fullf = fb + 4 <= rows;
      const int validf = (int)max<int64_t>(0, min<int64_t>(4, rows - fb));
      float v[8][4];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t c = c0 + 16 * i + tr;
        if (c < cols && fullf) {
          const float4 a = *reinterpret_cast<const float4 *>(x + c * ld + fb);
          v[i][0] = a.x; v[i][1] = a.y; v[i][2] = a.z; v[i][3] = a.w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[i][e] = (c < cols && e < validf) ? x[c * ld + fb + e] : 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) tile[tile_col(4 * fc + e, 16 * i + tr)] = v[i][e];
    }
    __syncthreads();

    // ---- phase 2: each thread owns tokens [32p, 32p+32) of feature fl ----
    float v[32];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const float4 a = *reinterpret_cast<const float4 *>(&tile[tile_col(fl, 32 * p + 4 * m)]);
      v[4 * m] = a.x; v[4 * m + 1] = a.y; v[4 * m + 2] = a.z; v[4 * m + 3] = a.w;
    }
    uint32_t am = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) am = max(am, abs_bits(v[e]));
    if constexpr (GRAN == 128) am = group_max_u32<4>(am);
    const GroupScale gs = group_scale<kUe8m0>(__uint_as_float(am));
    uint32_t w[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
      w[m] = e4m3x4(v[4 * m] * gs.mult, v[4 * m + 1] * gs.mult, v[4 * m + 2] * gs.mult,
                    v[4 * m + 3] * gs.mult);
    const int64_t cp = c0 + 32 * p;  // first token of this thread
    if (f < rows && cp < cols) {
      uint8_t *qp = q + f * q_ld + cp;
      if (cp + 32 <= cols) {
        reinterpret_cast<uint4 *>(qp)[0] = make_uint4(w[0], w[1], w[2], w[3]);
        reinterpret_cast<uint4 *>(qp)[1] = make_uint4(w[4], w[5], w[6], w[7]);
      } else {
        const int valid = (int)(cols - cp);
#pragma unroll
        for (int e = 0; e < 32; ++e)
          if (e < valid) qp[e] = (uint8_t)((w[e >> 2] >> (8 * (e & 3))) & 0xFFu);
      }
    }
    if constexpr (FMT != kSfPackedUe8m0) {
      float *sp = reinterpret_cast<float *>(sf);
      if (f < rows) {
        if constexpr (GRAN == 128) {
          if (p == 0) sp[f * sf_s_row + (c0 / 128) * sf_s_grp] = gs.sf;
        } else {
          if (cp < cols) sp[f * sf_s_row + (cp / 32) * sf_s_grp] = gs.sf;
        }
      }
    } else if constexpr (GRAN == 32) {
      // the 4 groups of this tile form one word; part p is group 4w + p
      const uint32_t mine = cp < cols ? gs.e8 << (8 * p) : 0u;
      const uint32_t word = group_or_u32<4>(mine);
      if (p == 0 && f < rows) reinterpret_cast<uint32_t *>(sf)[f * sf_s_row + (c0 / 128) * sf_s_grp] = word;
    } else {
      word128 |= gs.e8 << (8 * it);
    }
    __syncthreads();  // the next tile overwrites the LDS tile
  }
  if constexpr (FMT == kSfPackedUe8m0 && GRAN == 128) {
    if (p == 0 && f < rows && cbase < cols)
      reinterpret_cast<uint32_t *>(sf)[f * sf_s_row + (cbase / 512) * sf_s_grp] = word128;
  }
}

// ---------------------------------------------------------------------------
// Per-block cast.  Workgroups are persistent: workgroup w casts 128x128 blocks
// w, w + G, w + 2G, ... (G = grid size), and the loads of its next block are in
// flight while the current one is reduced and stored.  Thread t owns 8
// consecutive rows [8(t>>4), 8(t>>4)+8) x 8 columns [8(t&15), 8(t&15)+8) of a
// block: each load instruction covers 4 rows of 256 contiguous bytes.  The
// block amax is a DPP + LDS reduction.  Row-major E4M3 bytes leave as 8-byte
// stores; the optional transposed copy is an 8x8 byte transpose in registers,
// whose column k (8 consecutive rows) is one 8-byte store into row k of q^T.
// ---------------------------------------------------------------------------
template <typename TIn>
struct BlockRaw {   // a thread's 8 x 8 elements of one block, as loaded
  Raw16<TIn> r[4];  // rows 2p, 2p+1 of the 8 in r[p] (8 elements each)
};

template <typename TIn>
__device__ __forceinline__ void block_load(const TIn *x, int64_t rows, int64_t cols, int64_t x_ld, int64_t rb,
                                           int64_t c, BlockRaw<TIn> &br) {
  const int colvalid = (int)max<int64_t>(0, min<int64_t>(8, cols - c));
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t r = rb + 2 * p + h;
      constexpr int W = Raw16<TIn>::kWords / 2;   // words per 8 elements
      const int o = W * h;
      if (r < rows && colvalid == 8) {
        const TIn *src = x + r * x_ld + c;
#pragma unroll
        for (int i = 0; i < W / 4; ++i) {
          const uint4 v = reinterpret_cast<const uint4 *>(src)[i];
          br.r[p].w[o + 4 * i] = v.x; br.r[p].w[o + 4 * i + 1] = v.y;
          br.r[p].w[o + 4 * i + 2] = v.z; br.r[p].w[o + 4 * i + 3] = v.w;
        }
      } else {
        const bool any = r < rows && colvalid > 0;
        const TIn *src = x + (any ? r * x_ld + c : 0);
#pragma unroll
        for (int i = 0; i < W; ++i) br.r[p].w[o + i] = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (any && e < colvalid) {
            if constexpr (sizeof(TIn) == 2) br.r[p].w[o + (e >> 1)] |= (uint32_t)src[e] << (16 * (e & 1));
            else br.r[p].w[o + e] = __float_as_uint(src[e]);
          }
        }
      }
    }
  }
}

template <typename TIn, bool UE8M0, bool TRANS>
__global__ __launch_bounds__(kThreads) void cast_block_kernel(
    const TIn *__restrict__ x, int64_t rows, int64_t cols, int64_t x_ld, int64_t tiles_c, int64_t tiles,
    uint8_t *__restrict__ q, int64_t q_ld, float *__restrict__ sf, int64_t sf_ld, uint8_t *__restrict__ qT,
    int64_t qT_ld, float *__restrict__ sfT, int64_t sfT_ld) {
  __shared__ uint32_t red[2][kThreads / kWave];
  const int t = threadIdx.x;
  const int cc = t & 15, rg = t >> 4;
  BlockRaw<TIn> cur, nxt;
  int64_t blk = blockIdx.x;
  if (blk >= tiles) return;   // uniform over the workgroup
  block_load<TIn>(x, rows, cols, x_ld, (blk / tiles_c) * 128 + 8 * rg, (blk % tiles_c) * 128 + 8 * cc, cur);
  for (int it = 0; blk < tiles; ++it, blk += gridDim.x) {
    const int64_t bi = blk / tiles_c, bj = blk % tiles_c;
    const int64_t r0 = bi * 128, c0 = bj * 128;
    const int64_t c = c0 + 8 * cc, rb = r0 + 8 * rg;
    const int colvalid = (int)max<int64_t>(0, min<int64_t>(8, cols - c));
    const int64_t nblk = blk + gridDim.x;
    if (nblk < tiles)
      block_load<TIn>(x, rows, cols, x_ld, (nblk / tiles_c) * 128 + 8 * rg, (nblk % tiles_c) * 128 + 8 * cc, nxt);

    uint32_t am = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int e = 0; e < 16; ++e) am = max(am, abs_bits(cur.r[p].get(e)));
    am = wave_max_u32(am);
    uint32_t *rd = red[it & 1];   // alternate buffers: no second barrier before the next block
    if ((t & 63) == 0) rd[t >> 6] = am;
    __syncthreads();
    am = max(max(rd[0], rd[1]), max(rd[2], rd[3]));
    const GroupScale gs = group_scale<UE8M0>(__uint_as_float(am));

    uint32_t w[8][2];   // row i: columns 0-3, 4-7
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const Raw16<TIn> &rr = cur.r[i >> 1];
      const int o = 8 * (i & 1);
      w[i][0] = e4m3x4(rr.get(o) * gs.mult, rr.get(o + 1) * gs.mult, rr.get(o + 2) * gs.mult, rr.get(o + 3) * gs.mult);
      w[i][1] = e4m3x4(rr.get(o + 4) * gs.mult, rr.get(o + 5) * gs.mult, rr.get(o + 6) * gs.mult,
                       rr.get(o + 7) * gs.mult);
      const int64_t r = rb + i;
      if (r < rows && colvalid > 0) {
        uint8_t *qp = q + r * q_ld + c;
        if (colvalid == 8) {
          *reinterpret_cast<uint2 *>(qp) = make_uint2(w[i][0], w[i][1]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < colvalid) qp[e] = (uint8_t)((w[i][e >> 2] >> (8 * (e & 3))) & 0xFFu);
        }
      }
    }
    if (t == 0) {
      sf[bi * sf_ld + bj] = gs.sf;
      if constexpr (TRANS) sfT[bj * sfT_ld + bi] = gs.sf;
    }
    if constexpr (TRANS) {
      const int rvalid = (int)max<int64_t>(0, min<int64_t>(8, rows - rb));
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        if (k >= colvalid || rvalid == 0) continue;
        // byte k of every row: rows 0-3 -> lo, rows 4-7 -> hi
        const int sh = 8 * (k & 3), wi = k >> 2;
        const uint32_t lo = ((w[0][wi] >> sh) & 0xFFu) | (((w[1][wi] >> sh) & 0xFFu) << 8) |
                            (((w[2][wi] >> sh) & 0xFFu) << 16) | (((w[3][wi] >> sh) & 0xFFu) << 24);
        const uint32_t hi = ((w[4][wi] >> sh) & 0xFFu) | (((w[5][wi] >> sh) & 0xFFu) << 8) |
                            (((w[6][wi] >> sh) & 0xFFu) << 16) | (((w[7][wi] >> sh) & 0xFFu) << 24);
        uint8_t *op = qT + (c + k) * qT_ld + rb;
        if (rvalid == 8) {
          *reinterpret_cast<uint2 *>(op) = make_uint2(lo, hi);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < rvalid) op[e] = (uint8_t)((((e < 4) ? lo : hi) >> (8 * (e & 3))) & 0xFFu);
        }
      }
    }
    cur = nxt;
  }
}

// ---------------------------------------------------------------------------
// Dual-orientation per-token cast of a bf16 [rows, cols] matrix: the row-wise
// cast (1 x GRAN groups along cols) and the cast of its transpose (1 x GRAN
// groups along rows: the layout of the weight-gradient operands) from one read
// of x.  A 128x128 tile holds whole groups in both directions; one workgroup
// per tile.  GRAN is 128 or 32; FMT is fp32, UE8M0 or packed UE8M0 scales.
// Phase 1: lane (c = lane&15, j = lane>>4) of wave w loads columns [8c, 8c+8)
// of tile rows 32w + 2(4i+j) + s (i < 4, s < 2) with 16-byte loads (4 rows of
// 256 bytes per instruction); a 16-lane (GRAN 128) or 4-lane (GRAN 32) DPP max
// gives each group's amax and the row's E4M3 bytes leave as 8-byte stores.  The
// bf16 pairs of rows (2v, 2v+1) go to an LDS tile stored column-major (64
// words per column) at word v ^ 4h(col), h(f) = ((f>>3)^(f&3))&15.  Phase 2:
// thread t owns columns t>>2 and 64+(t>>2), rows [32p, 32p+32) with p = t&3;
// a 4-lane max (GRAN 128) or the thread's own 32 values (GRAN 32) give the
// amax, and the column's E4M3 bytes leave as two 16-byte stores.
// Packed UE8M0 words hold the exponent bytes of groups 4w..4w+3 (unused bytes
// zero): with GRAN 32 one word covers a tile's 128 columns (rows) and is
// assembled with a DPP OR; with GRAN 128 a word spans four tiles, so each tile
// stores its own byte, and the tile of the last group also zeroes the word's
// unused bytes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int dual_word(int f, int v) { return f * 64 + (v ^ (4 * (((f >> 3) ^ (f & 3)) & 15))); }
// fp32 input: one row per word, 128 words per column, the same key at 16-byte grain
__device__ __forceinline__ int dual_word32(int f, int r) { return f * 128 + (r ^ (4 * (((f >> 3) ^ (f & 3)) & 15))); }

template <int FMT>
__device__ __forceinline__ void store_scale(void *sf, int64_t idx, const GroupScale &gs) {
  reinterpret_cast<float *>(sf)[idx] = gs.sf;
}

// GRAN 128 packed: byte g%4 of word (row, g/4); the last group's tile zeroes the rest.
__device__ __forceinline__ void store_packed_byte(void *sf, int64_t row_off, int64_t s_grp, int64_t g, int64_t G,
                                                  uint32_t e8) {
  uint8_t *w = reinterpret_cast<uint8_t *>(reinterpret_cast<uint32_t *>(sf) + row_off + (g >> 2) * s_grp);
  w[g & 3] = (uint8_t)e8;
  if (g == G - 1)
    for (int b = (int)(g & 3) + 1; b < 4; ++b) w[b] = 0;
}

template <typename TIn, int GRAN, int FMT>
__global__ __launch_bounds__(kThreads) void cast_dual_kernel(
    const TIn *__restrict__ x, int64_t rows, int64_t cols, int64_t ld, int64_t tiles_c,
    uint8_t *__restrict__ q, int64_t q_ld, void *__restrict__ sf, int64_t sf_s_row, int64_t sf_s_grp,
    uint8_t *__restrict__ qT, int64_t qT_ld, void *__restrict__ sfT, int64_t sfT_s_row, int64_t sfT_s_grp) {
  static_assert(GRAN == 32 || GRAN == 128, "group 32 or 128");
  constexpr bool UE8M0 = FMT != kSfFp32;
  constexpr bool PACKED = FMT == kSfPackedUe8m0;
  constexpr bool F32 = sizeof(TIn) == 4;   // fp32 input: 8 words per 8 columns, one row per LDS word
  constexpr int W = F32 ? 8 : 4;
  __shared__ __attribute__((aligned(16))) uint32_t tile[F32 ? 128 * 128 : 128 * 64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * 128, c0 = (int64_t)(blockIdx.x % tiles_c) * 128;
  const int c = lane & 15, j = lane >> 4;
  const int64_t fc = c0 + 8 * c;
  const int validf = (int)max<int64_t>(0, min<int64_t>(8, cols - fc));
  const int64_t G = (cols + GRAN - 1) / GRAN, GT = (rows + GRAN - 1) / GRAN;   // groups per row / column

  uint32_t raw[4][2][W];   // bf16: column pairs; fp32: one column per word
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t r = r0 + 32 * wv + 2 * (4 * i + j) + s;
      uint32_t w[W];
#pragma unroll
      for (int k = 0; k < W; ++k) w[k] = 0u;
      if (r < rows && validf > 0) {
        const TIn *p = x + r * ld + fc;
        if (validf == 8) {
#pragma unroll
          for (int h = 0; h < W / 4; ++h) {
            const uint4 v = reinterpret_cast<const uint4 *>(p)[h];
            w[4 * h] = v.x; w[4 * h + 1] = v.y; w[4 * h + 2] = v.z; w[4 * h + 3] = v.w;
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < validf) {
              if constexpr (F32) w[e] = __float_as_uint(p[e]);
              else w[e >> 1] |= (uint32_t)p[e] << (16 * (e & 1));
            }
        }
      }
#pragma unroll
      for (int k = 0; k < W; ++k) raw[i][s][k] = w[k];
    }

  // rows: 1 x GRAN groups along the tile row (16 lanes x 8 columns, or 4 lanes per group)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (F32) v[e] = __uint_as_float(raw[i][s][e]);
        else v[e] = (e & 1) ? bf16_hi(raw[i][s][e >> 1]) : bf16_lo(raw[i][s][e >> 1]);
      }
      uint32_t am = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) am = max(am, abs_bits(v[e]));
      am = group_max_u32<GRAN / 8>(am);
      const GroupScale gs = group_scale<UE8M0>(__uint_as_float(am));
      const uint32_t w0 = e4m3x4(v[0] * gs.mult, v[1] * gs.mult, v[2] * gs.mult, v[3] * gs.mult);
      const uint32_t w1 = e4m3x4(v[4] * gs.mult, v[5] * gs.mult, v[6] * gs.mult, v[7] * gs.mult);
      const int64_t r = r0 + 32 * wv + 2 * (4 * i + j) + s;
      // group of this lane's columns, and the packed word of the tile row (GRAN 32)
      const int64_t g = (c0 + 8 * c) / GRAN;
      uint32_t word = 0;
      if constexpr (PACKED && GRAN == 32) {
        word = ((c & 3) == 0 && g < G) ? gs.e8 << (8 * ((c >> 2) & 3)) : 0u;
        word = group_or_u32<16>(word);
      }
      if (r < rows) {
        if (validf == 8) {
          *reinterpret_cast<uint2 *>(q + r * q_ld + fc) = make_uint2(w0, w1);
        } else if (validf > 0) {
          uint8_t *qp = q + r * q_ld + fc;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e < validf) qp[e] = (uint8_t)((((e < 4) ? w0 : w1) >> (8 * (e & 3))) & 0xFFu);
        }
        if constexpr (!PACKED) {
          if ((c & (GRAN / 8 - 1)) == 0 && g < G) store_scale<FMT>(sf, r * sf_s_row + g * sf_s_grp, gs);
        } else if constexpr (GRAN == 32) {
          if (c == 0) reinterpret_cast<uint32_t *>(sf)[r * sf_s_row + (c0 >> 7) * sf_s_grp] = word;
        } else {
          if (c == 0) store_packed_byte(sf, r * sf_s_row, sf_s_grp, c0 >> 7, G, gs.e8);
        }
      }
    }

  // transpose through LDS: bf16, word (col f, pair v) = rows 2v (low) and 2v+1 (high);
  // fp32, word (col f, row r)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int v = 16 * wv + 4 * i + j;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (F32) {
        tile[dual_word32(8 * c + e, 2 * v)] = raw[i][0][e];
        tile[dual_word32(8 * c + e, 2 * v + 1)] = raw[i][1][e];
      } else {
        const uint32_t lo = (raw[i][0][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const uint32_t hi = (raw[i][1][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        tile[dual_word(8 * c + e, v)] = lo | (hi << 16);
      }
    }
  }
  __syncthreads();

  // columns: 1 x GRAN groups along the tile column (4 lanes x 32 rows, or one lane's 32)
  const int p = t & 3;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int fl = (t >> 2) + 64 * half;
    float v[32];
    if constexpr (F32) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const uint4 a = *reinterpret_cast<const uint4 *>(&tile[dual_word32(fl, 32 * p + 4 * k)]);
        v[4 * k] = __uint_as_float(a.x); v[4 * k + 1] = __uint_as_float(a.y);
        v[4 * k + 2] = __uint_as_float(a.z); v[4 * k + 3] = __uint_as_float(a.w);
      }
    } else {
      uint32_t wd[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint4 a = *reinterpret_cast<const uint4 *>(&tile[dual_word(fl, 16 * p + 4 * k)]);
        wd[4 * k] = a.x; wd[4 * k + 1] = a.y; wd[4 * k + 2] = a.z; wd[4 * k + 3] = a.w;
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        v[2 * k] = bf16_lo(wd[k]);
        v[2 * k + 1] = bf16_hi(wd[k]);
      }
    }
    uint32_t am = 0;
#pragma unroll
    for (int e = 0; e < 32; ++e) am = max(am, abs_bits(v[e]));
    if constexpr (GRAN == 128) am = group_max_u32<4>(am);
    const GroupScale gs = group_scale<UE8M0>(__uint_as_float(am));
    uint32_t o[8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
      o[m] = e4m3x4(v[4 * m] * gs.mult, v[4 * m + 1] * gs.mult, v[4 * m + 2] * gs.mult, v[4 * m + 3] * gs.mult);
    const int64_t f = c0 + fl, tk = r0 + 32 * p;
    const int64_t gt = tk / GRAN;   // this thread's token group (GRAN 32), or the tile's (GRAN 128)
    uint32_t word = 0;
    if constexpr (PACKED && GRAN == 32) {
      word = gt < GT ? gs.e8 << (8 * p) : 0u;
      word = group_or_u32<4>(word);
    }
    if (f < cols) {
      if (tk < rows) {
        uint8_t *qp = qT + f * qT_ld + tk;
        if (tk + 32 <= rows) {
          reinterpret_cast<uint4 *>(qp)[0] = make_uint4(o[0], o[1], o[2], o[3]);
          reinterpret_cast<uint4 *>(qp)[1] = make_uint4(o[4], o[5], o[6], o[7]);
        } else {
          const int valid = (int)(rows - tk);
#pragma unroll
          for (int e = 0; e < 32; ++e)
            if (e < valid) qp[e] = (uint8_t)((o[e >> 2] >> (8 * (e & 3))) & 0xFFu);
        }
      }
      if constexpr (!PACKED) {
        if ((GRAN == 32 || p == 0) && gt < GT) store_scale<FMT>(sfT, f * sfT_s_row + gt * sfT_s_grp, gs);
      } else if constexpr (GRAN == 32) {
        if (p == 0) reinterpret_cast<uint32_t *>(sfT)[f * sfT_s_row + (r0 >> 7) * sfT_s_grp] = word;
      } else {
        if (p == 0) store_packed_byte(sfT, f * sfT_s_row, sfT_s_grp, r0 >> 7, GT, gs.e8);
      }
    }
  }
}

// Workgroups of `kernel` (256 threads) resident per CU, and the CU count, as
// the runtime reports them; callers keep the result in a function-local static
// of their own (one query per kernel, thread-safe initialisation).
struct Residency {
  int per_cu, cus;
};
template <typename K>
Residency residency(K kernel) {
  int dev = 0, n = 0, c = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kThreads, 0) != hipSuccess || n < 1 || c < 1)
    return Residency{2, 256};
  return Residency{n, c};
}

// Grid of a persistent kernel: all resident workgroups, at most `work`.
inline unsigned persistent_grid(const Residency &r, int64_t work) {
  const int64_t g = (int64_t)r.per_cu * r.cus;
  return (unsigned)(work < g ? work : g);
}

template <typename TIn, int GRAN, int FMT>
hipError_t launch_tok_rows(const void *x, int64_t rows, int64_t cols, int64_t xs_row, uint8_t *q,
                           int64_t q_ld, void *sf, int64_t sf_s_row, int64_t sf_s_grp, hipStream_t st) {
  const int64_t steps = (cols + kTokSpan - 1) / kTokSpan;
  // MN-major scales with 16-byte aligned columns of 4 rows: row-quad task order,
  // when there are enough tasks (>= 8192) that batches of four still leave 2048
  // waves; a small cast runs one task per wave instead (measured on MI355X,
  // 7..512 tokens x 4096: 3.8-4.3 us in row quads, 2.5-3.1 us one task per wave;
  // 3000 and 4096 tokens: row quads 10% faster)
  const bool quad = sf_s_row == 1 && sf_s_grp % 4 == 0 && reinterpret_cast<uintptr_t>(sf) % 16 == 0 && rows > 1 &&
                    rows * steps >= 8192;
  const int64_t tasks = quad ? (rows + 3) / 4 * 4 * steps : rows * steps;
  const int64_t target_waves = 16384;  // 16 waves per CU in flight
  int64_t tpw = (tasks + target_waves - 1) / target_waves;
  if (tpw < 1) tpw = 1;
  if (quad) tpw = (tpw + 3) / 4 * 4;   // whole batches of one row quad
  const int64_t waves = (tasks + tpw - 1) / tpw;
  // whole runs of 64 workgroups for the XCD-grouped numbering; a small cast
  // launches only the workgroups it needs
  const int64_t wgs = (waves + 3) / 4;
  const int64_t blocks = wgs < 64 ? wgs : (wgs + 63) / 64 * 64;
  const bool q16 = (reinterpret_cast<uintptr_t>(q) % 16 == 0) && (q_ld % 16 == 0);
#define FGFP8_ROWS(Q, QD)                                                                                         \
  hipLaunchKernelGGL((cast_tok_rows_kernel<TIn, GRAN, FMT, Q, QD>), dim3((unsigned)blocks), dim3(kThreads), 0, st, \
                     reinterpret_cast<const TIn *>(x), rows, cols, xs_row, q, q_ld, sf, sf_s_row, sf_s_grp, steps, \
                     tasks, tpw)
  if (quad) {
    if (q16) FGFP8_ROWS(true, true);
    else FGFP8_ROWS(false, true);
  } else {
    if (q16) FGFP8_ROWS(true, false);
    else FGFP8_ROWS(false, false);
  }
#undef FGFP8_ROWS
  return hipGetLastError();
}

template <typename TIn, int GRAN, int FMT>
hipError_t launch_tok_cols(const void *x, int64_t rows, int64_t cols, int64_t ld, uint8_t *q, int64_t q_ld,
                           void *sf, int64_t sf_s_row, int64_t sf_s_grp, hipStream_t st) {
  constexpr int NT = (FMT == kSfPackedUe8m0 && GRAN == 128) ? 4 : 1;
  const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((cols + 128 * NT - 1) / (128 * NT)));
  hipLaunchKernelGGL((cast_tok_cols_kernel<TIn, GRAN, FMT>), grid, dim3(kThreads), 0, st,
                     reinterpret_cast<const TIn *>(x), rows, cols, ld, q, q_ld, sf, sf_s_row, sf_s_grp);
  return hipGetLastError();
}

template <typename TIn>
hipError_t dispatch_tok(bool transposed, int gran, int fmt, const void *x, int64_t rows, int64_t cols,
                        int64_t xs, uint8_t *q, int64_t q_ld, void *sf, int64_t s_row, int64_t s_grp,
                        hipStream_t st) {
#define FGFP8_TOK(G, F)                                                                          \
  if (gran == G && fmt == F)                                                                     \
    return transposed ? launch_tok_cols<TIn, G, F>(x, rows, cols, xs, q, q_ld, sf, s_row, s_grp, st) \
                      : launch_tok_rows<TIn, G, F>(x, rows, cols, xs, q, q_ld, sf, s_row, s_grp, st);
  FGFP8_TOK(128, kSfFp32)
  FGFP8_TOK(128, kSfUe8m0)
  FGFP8_TOK(128, kSfPackedUe8m0)
  FGFP8_TOK(32, kSfFp32)
  FGFP8_TOK(32, kSfUe8m0)
  FGFP8_TOK(32, kSfPackedUe8m0)
#undef FGFP8_TOK
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_cast_per_token(const CastTokenArgs &a, hipStream_t st) {
  const bool transposed = a.x_stride_col != 1;
  const int64_t xs = transposed ? a.x_stride_col : a.x_stride_row;
  if (a.x_dtype == kInBf16)
    return dispatch_tok<uint16_t>(transposed, a.gran_k, a.sf_fmt, a.x, a.rows, a.cols, xs, a.q, a.q_ld, a.sf,
                                  a.sf_stride_row, a.sf_stride_group, st);
  return dispatch_tok<float>(transposed, a.gran_k, a.sf_fmt, a.x, a.rows, a.cols, xs, a.q, a.q_ld, a.sf,
                             a.sf_stride_row, a.sf_stride_group, st);
}

hipError_t launch_cast_dual(const CastDualArgs &a, hipStream_t st) {
  const int64_t tiles_c = (a.cols + 127) / 128, tiles = tiles_c * ((a.rows + 127) / 128);
  const dim3 grid((unsigned)tiles);
#define FGFP8_DUAL(T, GR, F)                                                                                  \
  hipLaunchKernelGGL((cast_dual_kernel<T, GR, F>), grid, dim3(kThreads), 0, st, reinterpret_cast<const T *>(a.x), \
                     a.rows, a.cols, a.x_ld, tiles_c, a.q, a.q_ld, a.sf, a.sf_stride_row, a.sf_stride_group, a.qT,   \
                     a.qT_ld, a.sfT, a.sfT_stride_row, a.sfT_stride_group)
#define FGFP8_DUAL_FMT(T)                                                   \
  if (a.gran_k == 32) {                                                     \
    if (a.sf_fmt == kSfPackedUe8m0) FGFP8_DUAL(T, 32, kSfPackedUe8m0);      \
    else if (a.sf_fmt == kSfUe8m0) FGFP8_DUAL(T, 32, kSfUe8m0);             \
    else FGFP8_DUAL(T, 32, kSfFp32);                                        \
  } else {                                                                  \
    if (a.sf_fmt == kSfPackedUe8m0) FGFP8_DUAL(T, 128, kSfPackedUe8m0);     \
    else if (a.sf_fmt == kSfUe8m0) FGFP8_DUAL(T, 128, kSfUe8m0);            \
    else FGFP8_DUAL(T, 128, kSfFp32);                                       \
  }
  if (a.x_dtype == kInFp32) {
    FGFP8_DUAL_FMT(float)
  } else {
    FGFP8_DUAL_FMT(uint16_t)
  }
#undef FGFP8_DUAL_FMT
#undef FGFP8_DUAL
  return hipGetLastError();
}

hipError_t launch_cast_per_block(const CastBlockArgs &a, hipStream_t st) {
  // persistent workgroups, each walking blocks with the next one's loads in flight
  const int64_t tiles_c = (a.cols + 127) / 128, tiles = tiles_c * ((a.rows + 127) / 128);
  const bool ue = a.sf_fmt == kSfUe8m0;
  const bool tr = a.qT != nullptr;
#define FGFP8_BLK(T, U, TR)                                                                              \
  do {                                                                                                   \
    static const Residency res = residency(cast_block_kernel<T, U, TR>);                                \
  hipLaunchKernelGGL((cast_block_kernel<T, U, TR>), dim3(persistent_grid(res, tiles)), dim3(kThreads), 0, st, \
                     reinterpret_cast<const T *>(a.x), a.rows, a.cols, a.x_ld, tiles_c, tiles, a.q, a.q_ld, \
                     a.sf, a.sf_ld, a.qT, a.qT_ld, a.sfT, a.sfT_ld);                                   \
  } while (0)
  if (a.x_dtype == kInBf16) {
    if (ue) { if (tr) FGFP8_BLK(uint16_t, true, true); else FGFP8_BLK(uint16_t, true, false); }
    else    { if (tr) FGFP8_BLK(uint16_t, false, true); else FGFP8_BLK(uint16_t, false, false); }
  } else {
    if (ue) { if (tr) FGFP8_BLK(float, true, true); else FGFP8_BLK(float, true, false); }
    else    { if (tr) FGFP8_BLK(float, false, true); else FGFP8_BLK(float, false, false); }
  }
#undef FGFP8_BLK
  return hipGetLastError();
}

}  // namespace fgfp8
