// gemm.hip -- fine-grained block-scaled FP8 NT GEMM for gfx950.
//
// D = (A * sa)(B * sb)^T, A [m, k] and B [n, k] E4M3 row-major ("DeepGEMM
// Essentials: High-Performance FP8 Matrix Multiplication", Parts 1 and 6).
// Forward / dgrad: for every 128-wide K block one V_MFMA_SCALE_F32_16X16X128_F8F6F4
// (neutral hardware scales) per 16x16 output tile produces that block's partial
// sum, which is then promoted into an fp32 register accumulator with the
// fine-grained scales sa(i, kb) * sb(j/128, kb) (one RHS scale per 128x128
// block, whose row of ceil(k/128) values serves every K block -- the reply in
// "[Help] Starter script for nn.Linear for fwd,bwd").  Weight gradient
// ("DeepGEMM Essentials", Parts 12-13: fp32 output, accumulated in place):
// sa(i, kb) * sb(j, kb), with the block sums taken on the bf16 MFMA
// (gemm_wgrad_kernel explains why).
//
// gfx950 design notes (measured on MI355X):
//  * The FP8 MFMA sustains ~4.6 PF, but dependent fp32 VALU work issued right
//    after it serialises with it.  So the promotion of block kb-1's partial
//    sums is software-pipelined under block kb's MFMAs: each MFMA writes a
//    fresh partial P[t] that is consumed one K block later, and the issue
//    order is pinned MFMA by MFMA with sched_barrier.
//    (The MFMA results are kept in VGPRs: -mllvm --amdgpu-mfma-vgpr-form.)
//  * A and B K-tiles (128 bytes of K per row) are copied global -> LDS by
//    global_load_lds_dwordx4 (no VGPR staging), two stages deep.  Each lane
//    fetches the 16-byte chunk that belongs at its fixed LDS slot under a
//    16-byte XOR swizzle of the row's low bits (swz_key), so fragment reads
//    (ds_read_b128) are free of bank conflicts.
//  * 256 threads = 4 waves in a 2x2 grid over a 128x128 output tile, each
//    wave 64x64 = 4x4 MFMA tiles; 2 workgroups per CU.
//  * B is the MFMA's first operand, so a lane holds four consecutive output
//    columns of one row (8-byte bf16 stores, 16-byte fp32 read-modify-write).
//  * Workgroups are mapped XCD by XCD onto bands of 8 m-tiles so that the
//    tiles resident on one XCD share A and B panels in its L2.
//  * Operands that are not in the MALL stall the copies on HBM latency, which
//    the two stages cannot hide: the first round of workgroups reads all of B
//    once, and each weight-gradient tile reads its D, right after block 0's
//    copies (overlapped with block 0's MFMAs).
//  * Weight-gradient, decode-sized and UE8M0 variants follow below.
#include <algorithm>
#include <atomic>

#include "device_common.h"
#include "launch.h"
#include "tile_common.h"

namespace fgfp8 {
namespace {


// Tile configuration: WAVES_M x WAVES_N waves, each owning a 64x64 output block;
// STAGES LDS stages of (BM + BN) x 128 bytes.
template <int WAVES_M, int WAVES_N, int STAGES>
struct Cfg {
  static constexpr int kWaves = WAVES_M * WAVES_N;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kBM = 64 * WAVES_M, kBN = 64 * WAVES_N;
  static constexpr int kABytes = kBM * kBK, kBBytes = kBN * kBK;
  static constexpr int kSaOff = kABytes + kBBytes;          // BM fp32 (or packed word) row scales
  static constexpr int kSbOff = kSaOff + 4 * kBM;           // forward: 64 copies of one fp32; wgrad: BN fp32
  static constexpr int kSaLoads = kBM / 64;                 // 4-byte direct loads of 64 lanes
  static constexpr int kSbLoads = kBN / 64;
  static constexpr int kStageBytes = kSbOff + 4 * kBN;
  static constexpr int kALoads = kABytes / 1024 / kWaves;   // 1 KB direct loads per wave per stage
  static constexpr int kBLoads = kBBytes / 1024 / kWaves;
  static_assert(kALoads * 1024 * kWaves == kABytes && kBLoads * 1024 * kWaves == kBBytes, "tile split");
  static constexpr int kStages = STAGES;
  static constexpr int WAVES_N_ = WAVES_N;
  static constexpr int kMinBlocks = kWaves <= 4 ? 2 : 1;   // workgroups per CU the registers are sized for
};


// MFMA operand: lane l holds row (l & 15) and K bytes [32*(l>>4), 32*(l>>4)+32).
// A and B fragments use the same K mapping, so the product does not depend on
// which order the instruction assigns to the 128 K positions.
__device__ __forceinline__ v8i frag(const uint8_t *tile, int row, int lane) {
  const int c = (lane >> 4) << 1;
  const u32x4 lo = *reinterpret_cast<const u32x4 *>(tile + swz(row, c));
  const u32x4 hi = *reinterpret_cast<const u32x4 *>(tile + swz(row, c + 1));
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// 16x16 outputs, K = 128, fp32 result, E4M3 x E4M3, hardware scales 2^0.
__device__ __forceinline__ v4f mfma_k128(v8i a, v8i b) {
  const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 127, 0, 127);
}


template <int SA_FMT>
__device__ __forceinline__ float load_sa(const void *sa, int64_t sa_ld, int64_t i, int kb) {
  if constexpr (SA_FMT == kSfPackedUe8m0) {
    const uint32_t w = reinterpret_cast<const uint32_t *>(sa)[(int64_t)(kb >> 2) * sa_ld + i];
    return __uint_as_float(((w >> (8 * (kb & 3))) & 0xFFu) << 23);
  } else {
    return reinterpret_cast<const float *>(sa)[(int64_t)kb * sa_ld + i];
  }
}

// Scales of one K block as the forward / dgrad promotion uses them.
struct BlockScales {
  float sa[4];      // per row-subtile (the lane's row)
  float sb;         // uniform over the wave's 64 columns (one 128x128 block of B)
};


// B prefetch of one workgroup of the first round (blockIdx.x < b_prefetch_wgs):
// its share of B's 1 KB row chunks, up to kPrefetch copies per wave (64 KB per
// workgroup; chunks past the share repeat its last one), into the 1 KB slot
// `junk`.  Exactly kPrefetch copies per wave, so the first wait can count them.
constexpr int kPrefetch = 16;
template <class C>
__device__ __forceinline__ void b_prefetch(const GemmArgs &g, int64_t n, int wv, int lane, uint8_t *junk) {
  const int64_t per_row = (g.k + 1023) / 1024, total = n * per_row;   // total >= 1
  const int64_t per_wg = (total + g.b_prefetch_wgs - 1) / g.b_prefetch_wgs;
  const int64_t c_first = (int64_t)blockIdx.x * per_wg;
  const int64_t c_last = min(c_first + per_wg, total) - 1;   // may lie below c_first: then the last chunk
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j) {
    const int64_t c = min(c_first + wv + (int64_t)j * C::kWaves, c_last);
    const int64_t row = c / per_row;
    const uint32_t col = (uint32_t)min((c - row * per_row) * 1024 + 16 * lane, g.k - 16);
    load_lds16(g.B + row * g.ldb, col, junk);
  }
}

// D prefetch of a weight-gradient tile (fp32 D is read and added to at the end):
// the tile's 128 rows x 512 bytes as 64 copies of 1 KB (two rows each), exactly
// kPrefetch per wave of a 4-wave 128x128 tile, into the 1 KB slot `junk`, so that
// the epilogue's read of D finds it in the caches.  Interior tiles only (nothing
// outside D is read), and only while the offsets fit 32 bits.
template <class C>
__device__ __forceinline__ bool d_prefetch(const GemmArgs &g, int64_t m0, int64_t n0, int wv, int lane,
                                           uint8_t *junk) {
  static_assert(C::kBM == 128 && C::kBN == 128 && C::kWaves * kPrefetch * 2 == C::kBM, "two rows per copy");
  if (m0 + C::kBM > g.m || n0 + C::kBN > g.n || g.ldd > ((int64_t)1 << 22)) return false;
  const float *dbase = reinterpret_cast<const float *>(g.D) + m0 * g.ldd + n0;
#pragma unroll
  for (int j = 0; j < kPrefetch; ++j) {
    const int r = 2 * (wv + C::kWaves * j) + (lane >> 5);
    load_lds16(dbase, (uint32_t)((int64_t)r * g.ldd * 4 + (lane & 31) * 16), junk);
  }
  return true;
}

// acc += P * sa(i, kb) * sb(j/128, kb) for an MFMA tile of row-subtile mi
__device__ __forceinline__ void promote(v4f &acc, const v4f &p, const BlockScales &s, int mi) {
  const float c = s.sa[mi] * s.sb;
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r] = __builtin_fmaf(p[r], c, acc[r]);
}



// Direct-to-LDS copies of the A and B tiles of one K block (128 bytes of K per
// row).  Offsets are 32-bit from the tile's first row (the host bounds lda, ldb
// below 2^24).  Each 1 KB wave instruction fills 64 consecutive 16-byte slots:
// slot s holds row s/8, physical chunk s%8, i.e. logical chunk (s%8) ^
// swz_key(row).  Wave wv issues tile instructions wv, wv + kWaves, ...; rows past
// the matrix edge read its last row (their results are never stored).  The scale
// rows (4 bytes per lane) are spread over the first waves: sa's kBM rows, then
// sb's kBN columns (or its one block scale).
template <class C>
struct TileCopy {
  uint32_t a_off[C::kALoads], b_off[C::kBLoads];
  bool sa_loader, sb_loader;
  uint32_t scale_off;   // row of sa (or column of sb) this lane copies, times 4

  __device__ __forceinline__ TileCopy(const GemmArgs &g, int64_t m0, int64_t n0, int wv, int lane) {
#pragma unroll
    for (int i = 0; i < C::kALoads; ++i) {
      const int s = 64 * (i * C::kWaves + wv) + lane, row = s >> 3, chunk = (s & 7) ^ swz_key(row);
      a_off[i] = (uint32_t)(min((int64_t)row, g.m - 1 - m0) * g.lda) + (uint32_t)(chunk * 16);
    }
#pragma unroll
    for (int i = 0; i < C::kBLoads; ++i) {
      const int s = 64 * (i * C::kWaves + wv) + lane, row = s >> 3, chunk = (s & 7) ^ swz_key(row);
      b_off[i] = (uint32_t)(min((int64_t)row, g.n - 1 - n0) * g.ldb) + (uint32_t)(chunk * 16);
    }
    static_assert(C::kSaLoads + C::kSbLoads <= C::kWaves, "one scale load per wave at most");
    sa_loader = wv < C::kSaLoads;
    sb_loader = wv >= C::kSaLoads && wv < C::kSaLoads + C::kSbLoads;
    scale_off = sa_loader ? 4u * (uint32_t)min((int64_t)(64 * wv + lane), g.m - 1 - m0)
                          : 4u * (uint32_t)min((int64_t)(64 * (wv - C::kSaLoads) + lane), g.n - 1 - n0);
  }
  // tiles of the K block whose first bytes are ga (row m0 of A) and gb (row n0 of B)
  __device__ __forceinline__ void tiles(const uint8_t *ga, const uint8_t *gb, uint8_t *st, int wv) const {
#pragma unroll
    for (int i = 0; i < C::kALoads; ++i) load_lds16(ga, a_off[i], st + 1024 * (i * C::kWaves + wv));
#pragma unroll
    for (int i = 0; i < C::kBLoads; ++i) load_lds16(gb, b_off[i], st + C::kABytes + 1024 * (i * C::kWaves + wv));
  }
  // the scale dwords of the stage: sa_row = &sa(m0, kb) (MN-major), sb_row = &sb(n0, kb)
  // (MN-major, one per column) or the block scale itself (block_sb: every lane copies it)
  __device__ __forceinline__ void scales(const void *sa_row, const void *sb_row, bool block_sb, uint8_t *st,
                                         int wv) const {
    if (sa_loader)
      load_lds4(sa_row, scale_off, st + C::kSaOff + 256 * wv);
    else if (sb_loader)
      load_lds4(sb_row, block_sb ? 0u : scale_off, st + C::kSbOff + 256 * (wv - C::kSaLoads));
  }
};

// Weight-gradient epilogue: D += acc in fp32 for the wave's 64x64 block, a lane
// holding row i, columns j..j+3 of each 16x16 tile (16-byte read-modify-write).
__device__ __forceinline__ void wgrad_store(const GemmArgs &g, const v4f (&acc)[16], int64_t m0, int64_t n0,
                                            int wm, int wn, int lane) {
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int64_t i = m0 + wm + 16 * mi + (lane & 15);
    if (i >= g.m) continue;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t j = n0 + wn + 16 * ni + 4 * (lane >> 4);
      if (j >= g.n) continue;
      const v4f a = acc[4 * mi + ni];
      float *dp = reinterpret_cast<float *>(g.D) + i * g.ldd + j;
      if (j + 4 <= g.n) {
        const v4f d = *reinterpret_cast<const v4f *>(dp);
        *reinterpret_cast<v4f *>(dp) = d + a;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j + r < g.n) dp[r] += a[r];
      }
    }
  }
}

// Per-token cast of the bf16 output fused into the epilogue: the 128 columns of a
// tile row are exactly one 1x128 group ("DeepGEMM Essentials", Part 3: amax,
// clamp, scale amax/448, E4M3), taken over the bf16-rounded values so that
// the result equals casting the stored bf16 output.  A lane holds 16 of a
// row's columns; the 4 lanes of that row in a wave (lane, lane^16, lane^32,
// lane^48) reduce with shuffles, and the two waves holding the row's two
// 64-column halves combine through LDS.
template <class C, bool UE8M0>
__device__ __forceinline__ void fused_cast_epilogue(const GemmArgs &g, const v4f (&acc)[16], int64_t m0, int64_t n0,
                                                    int wm, int wn, int lane) {
  static_assert(C::kBN == 128, "a tile row is one 128-column group");
  __shared__ uint32_t half_amax[2][C::kBM];
  const int64_t m = g.m, n = g.n;
  uint32_t am[4];
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    am[mi] = 0;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t j = n0 + wn + 16 * ni + 4 * (lane >> 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = __uint_as_float(bf16_rne(acc[4 * mi + ni][r]) << 16);
        if (j + r < n) am[mi] = max(am[mi], __float_as_uint(v) & 0x7FFFFFFFu);
      }
    }
    am[mi] = max(am[mi], (uint32_t)__shfl_xor((int)am[mi], 16));
    am[mi] = max(am[mi], (uint32_t)__shfl_xor((int)am[mi], 32));
  }
  if (lane < 16) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) half_amax[wn >> 6][wm + 16 * mi + lane] = am[mi];
  }
  __syncthreads();
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int row = wm + 16 * mi + (lane & 15);
    const int64_t i = m0 + row;
    const GroupScale gs = group_scale<UE8M0>(__uint_as_float(max(half_amax[0][row], half_amax[1][row])));
    if (i >= m) continue;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t j = n0 + wn + 16 * ni + 4 * (lane >> 4);
      if (j >= n) continue;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = __uint_as_float(bf16_rne(acc[4 * mi + ni][r]) << 16);
      const uint32_t w = e4m3x4(v[0] * gs.mult, v[1] * gs.mult, v[2] * gs.mult, v[3] * gs.mult);
      uint8_t *qp = g.q + i * g.q_ld + j;
      if (j + 4 <= n) {
        *reinterpret_cast<uint32_t *>(qp) = w;
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j + r < n) qp[r] = (uint8_t)((w >> (8 * r)) & 0xFFu);
      }
    }
    if (wn == 0 && (lane >> 4) == 0) g.cq_sf[i * g.cq_s_row + (n0 >> 7) * g.cq_s_grp] = gs.sf;
  }
}

// KSLICE: the workgroup takes K blocks [KB*y/Y, KB*(y+1)/Y) of its tile, y =
// blockIdx.y of Y = gridDim.y slices (the launcher keeps Y <= KB, so no slice is
// empty), and stores its promoted fp32 sums to the workspace instead of D.
template <class C, int SA_FMT, bool GROUPED, int CASTF, bool KSLICE = false>
__global__ __launch_bounds__(C::kThreads, C::kMinBlocks) void gemm_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  static_assert(!KSLICE || (!GROUPED && CASTF == 0), "K slices of plain tiles only");
  // the stages, then a 1 KB slot that receives the B prefetch copies
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kStages * C::kStageBytes + 1024];
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = (wv / C::WAVES_N_) * 64, wn = (wv % C::WAVES_N_) * 64;
  int64_t m0, n0;
  if (!tile_origin<C>(tiles_m, tiles_n, m0, n0)) return;
  const int64_t m = g.m, n = g.n;
  const int KB = (int)(g.k / kBK);
  int kb_lo = 0, kb_hi = KB;
  if constexpr (KSLICE) {
    kb_lo = (int)((int64_t)KB * blockIdx.y / gridDim.y);
    kb_hi = (int)((int64_t)KB * (blockIdx.y + 1) / gridDim.y);
    if (kb_lo >= kb_hi) return;   // not launched so; nothing issued yet
  }

  // m-grouped layout: the tile's 128 rows belong to one expert, the largest
  // m_indices among them (-1 marks padding); a tile with no valid expert id
  // writes nothing.  Every wave computes the same id, so the whole workgroup
  // returns together, before any barrier.
  const uint8_t *Bg = g.B;
  const float *sbg = g.sb;
  int expert = 0;
  if constexpr (GROUPED) {
    static_assert(C::kBM == 128, "one 128-row segment block per tile");
    uint32_t v = 0;
#pragma unroll
    for (int r = 0; r < C::kBM; r += 64)
      if (m0 + r + lane < m) v = max(v, (uint32_t)(g.m_idx[m0 + r + lane] + 1));
    expert = (int)wave_max_u32(v) - 1;
    if (expert < 0 || expert >= g.num_experts) return;
    Bg = g.B + (int64_t)expert * g.b_estride;
    sbg = g.sb + (int64_t)expert * g.sb_estride;
  }

  // One stage: the A and B tiles of K block kb, A's row scales (MN-major; packed
  // words hold four K blocks) and B's one block scale of the tile.
  const TileCopy<C> cp(g, m0, n0, wv, lane);
  auto issue = [&](int kb, uint8_t *st) {
    cp.tiles(g.A + m0 * g.lda + (int64_t)kb * kBK, Bg + n0 * g.ldb + (int64_t)kb * kBK, st, wv);
    const int64_t col = SA_FMT == kSfPackedUe8m0 ? (kb >> 2) : kb;
    cp.scales(reinterpret_cast<const uint32_t *>(g.sa) + col * g.sa_ld + m0, sbg + (n0 >> 7) * g.sb_ld + kb, true,
              st, wv);
  };
  auto read_scales = [&](int kb, const uint8_t *st, BlockScales &s) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const float v = *reinterpret_cast<const float *>(st + C::kSaOff + 4 * (wm + 16 * mi + (lane & 15)));
      if constexpr (SA_FMT == kSfPackedUe8m0) {
        s.sa[mi] = __uint_as_float(((__float_as_uint(v) >> (8 * (kb & 3))) & 0xFFu) << 23);
      } else {
        s.sa[mi] = v;
      }
    }
    s.sb = *reinterpret_cast<const float *>(st + C::kSbOff);
  };

  BlockScales prev;   // scales of the K block whose partial sums are pending
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) prev.sa[mi] = 0.0f;
  prev.sb = 0.0f;

  v4f acc[16], p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[i] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    p[i] = acc[i];
  }

  // Pipeline, two LDS stages; block kb lives in stage kb%2.  Step kb waits until
  // its stage has landed (its own copies, then a bare s_barrier for everyone's,
  // which also tells every wave that all reads of the other stage are done),
  // issues the copy of block kb+1 into the other stage, reads block kb's
  // fragments and scales and runs its MFMAs beside the promotion of block kb-1.
  // The wait and the barrier are inline assembly so that the fragment reads
  // cannot be scheduled above them; __syncthreads() is not used because its
  // fence would also wait for the copy in flight.  (Measured on MI355X: issuing
  // the copy of block kb+2 half-way through step kb behind a second barrier,
  // or prefetching the next block into L2, does not help: the copy path's
  // bytes per clock, not its latency, is the limit with 128x128 tiles.)
  static_assert(C::kStages == 2, "two stages");
  //
  // B prefetch.  The XCD tile order has all eight XCDs read the same B panels in
  // the same round of tiles, so a B that is not in the MALL (the 256 MB cache in
  // front of HBM) stalls every XCD's copies on HBM latency in every round, which
  // the two-stage pipeline cannot hide.  The first round of workgroups therefore
  // reads B once (b_prefetch: its share of up to 64 KB per workgroup) right after
  // block 0's copies: kPrefetch 1 KB copies per wave into the spare LDS slot.
  // Copies complete in order, so the first wait lets exactly those be in flight
  // and block 0's MFMAs overlap them.  Measured on MI355X in the linear step
  // (20 steps back to back): dgrad 291 -> 273 us (its B, W^T, was written long
  // before), forward +1%, step -1.4%.  The launcher enables it for grids of more
  // than one round only.
  issue(kb_lo, smem + (kb_lo & 1) * C::kStageBytes);
  const bool prefetching = !GROUPED && !KSLICE && (int)blockIdx.x < g.b_prefetch_wgs;
  if (prefetching) b_prefetch<C>(g, n, wv, lane, smem + C::kStages * C::kStageBytes);
  for (int kb = kb_lo; kb < kb_hi; ++kb) {
    // wave priority 0 while waiting and issuing copies, 3 once its MFMAs run (below):
    // the SIMD's other wave, if it is in its MFMA phase, is served first
    if (prefetching && kb == 0)   // block 0 has landed; the prefetch copies may be in flight
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n\ts_setprio 0" ::"n"(kPrefetch) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n\ts_setprio 0" ::: "memory");
    const uint8_t *st = smem + (kb & 1) * C::kStageBytes;
    // The copy into the free stage goes first: inline assembly bounds the
    // scheduling region, and the fragment reads must share one with the MFMAs.
    if (kb + 1 < kb_hi) issue(kb + 1, smem + ((kb + 1) & 1) * C::kStageBytes);
    BlockScales cur;
    read_scales(kb, st, cur);
    // Tiles run in a snake order (row 0 left to right, row 1 right to left, ...)
    // so that each MFMA needs at most one fragment beyond the previous ones.
    // Fragment read order: a0 b0 b1 | b2 | b3 | a1 | a2 | a3, each read at least two
    // MFMAs ahead of its first use (b1 at 1, b2 at 2, b3 at 3, a1 at 4, a2 at 8,
    // a3 at 12); sched_barrier pins this order (left alone, the scheduler hoists
    // every read above the first MFMA, which then waits for all of them).
    v8i af[4], bf[4];
    af[0] = frag(st, wm + (lane & 15), lane);
    bf[0] = frag(st + C::kABytes, wn + (lane & 15), lane);
    bf[1] = frag(st + C::kABytes, wn + 16 + (lane & 15), lane);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q < 2) bf[q + 2] = frag(st + C::kABytes, wn + 16 * (q + 2) + (lane & 15), lane);
      else if (q < 5) af[q - 1] = frag(st, wm + 16 * (q - 1) + (lane & 15), lane);
      const int mi = q >> 2, ni = (mi & 1) ? 3 - (q & 3) : (q & 3), i = 4 * mi + ni;
      // promote tile i of block kb-1 (scales `prev`) beside block kb's MFMA
      promote(acc[i], p[i], prev, mi);
      p[i] = mfma_k128(bf[ni], af[mi]);
      if (q == 0) __builtin_amdgcn_s_setprio(3);
      __builtin_amdgcn_sched_barrier(0);
    }
    prev = cur;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) promote(acc[i], p[i], prev, i >> 2);

  if constexpr (KSLICE) {
    // slot (tile, slice): per wave 16 x 64 lanes of v4f, each store 1 KB contiguous
    const int64_t tile = (m0 / C::kBM) * tiles_n + n0 / C::kBN;
    v4f *dst = reinterpret_cast<v4f *>(g.part) + ((tile * gridDim.y + blockIdx.y) * C::kWaves + wv) * 1024 + lane;
#pragma unroll
    for (int i = 0; i < 16; ++i) dst[i * 64] = acc[i];
    return;
  }

  // epilogue: lane holds row i, columns j..j+3 of every 16x16 tile
  if constexpr (CASTF != 0) fused_cast_epilogue<C, CASTF == 2>(g, acc, m0, n0, wm, wn, lane);
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int64_t i = m0 + wm + 16 * mi + (lane & 15);
    if (i >= m) continue;
    if constexpr (GROUPED) {
      if (g.m_idx[i] != expert) continue;   // padding (or another expert's) row
    }
    if constexpr (CASTF != 0) {
      if (g.D == nullptr) continue;         // only the FP8 output was asked for
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t j = n0 + wn + 16 * ni + 4 * (lane >> 4);
      if (j >= n) continue;
      const v4f a = acc[4 * mi + ni];
      uint16_t *dp = reinterpret_cast<uint16_t *>(g.D) + i * g.ldd + j;
      const uint32_t h0 = bf16_rne(a[0]) | (bf16_rne(a[1]) << 16);
      const uint32_t h1 = bf16_rne(a[2]) | (bf16_rne(a[3]) << 16);
      if (j + 4 <= n) {
        *reinterpret_cast<u32x2 *>(dp) = (u32x2){h0, h1};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j + r < n) dp[r] = (uint16_t)bf16_rne(a[r]);
      }
    }
  }
}

// Few tiles and a long K (m = 512 decode: 224 or 128 tiles of 128x128 for 256 CUs):
// there one workgroup's chain of K steps, about 0.85 us each whether a CU runs one
// workgroup or two, sets the time.  Here a workgroup of 8 waves runs two chains on
// one 128x128 tile: group g (waves 4g..4g+3, gemm_kernel's 2x2 wave layout) takes
// K blocks g, g+2, g+4, ... through its own two LDS stages, with gemm_kernel's
// copies, waits, fragment order and promotion; all 8 waves meet at each step's
// barrier.  At the end group 1's promoted sums go through LDS and group 0 adds them
// to its own (fixed order: the result is deterministic) and stores bf16.
template <class C, int SA_FMT>
__global__ __launch_bounds__(2 * C::kThreads, 1) void gemm_ksplit2_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  static_assert(C::kBM == 128 && C::kBN == 128 && C::kStages == 2, "128x128 tiles, two stages per group");
  static_assert(2 * C::kStages * C::kStageBytes >= C::kWaves * 16 * 64 * 16, "the reduction fits the stages");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * C::kStages * C::kStageBytes];
  const int t = threadIdx.x, lane = t & 63;
  const int wg8 = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = wg8 / C::kWaves, wv = wg8 % C::kWaves;
  const int wm = (wv / C::WAVES_N_) * 64, wn = (wv % C::WAVES_N_) * 64;
  int64_t m0, n0;
  if (!tile_origin<C>(tiles_m, tiles_n, m0, n0)) return;
  const int64_t m = g.m, n = g.n;
  const int KB = (int)(g.k / kBK);
  uint8_t *gs = smem + grp * C::kStages * C::kStageBytes;   // this group's two stages

  const TileCopy<C> cp(g, m0, n0, wv, lane);
  auto issue = [&](int kb, uint8_t *st) {
    cp.tiles(g.A + m0 * g.lda + (int64_t)kb * kBK, g.B + n0 * g.ldb + (int64_t)kb * kBK, st, wv);
    const int64_t col = SA_FMT == kSfPackedUe8m0 ? (kb >> 2) : kb;
    cp.scales(reinterpret_cast<const uint32_t *>(g.sa) + col * g.sa_ld + m0, g.sb + (n0 >> 7) * g.sb_ld + kb, true,
              st, wv);
  };
  auto read_scales = [&](int kb, const uint8_t *st, BlockScales &s) {
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) {
      const float v = *reinterpret_cast<const float *>(st + C::kSaOff + 4 * (wm + 16 * mi + (lane & 15)));
      if constexpr (SA_FMT == kSfPackedUe8m0) {
        s.sa[mi] = __uint_as_float(((__float_as_uint(v) >> (8 * (kb & 3))) & 0xFFu) << 23);
      } else {
        s.sa[mi] = v;
      }
    }
    s.sb = *reinterpret_cast<const float *>(st + C::kSbOff);
  };

  BlockScales prev;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) prev.sa[mi] = 0.0f;
  prev.sb = 0.0f;
  v4f acc[16], p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    acc[i] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    p[i] = acc[i];
  }

  // step s: group g's block kb = 2s + g lives in its stage s%2; a group whose block
  // is past K (group 1 in the last step of an odd KB) only meets the barrier
  const int steps = (KB + 1) / 2;
  if (grp < KB) issue(grp, gs);
  for (int s = 0; s < steps; ++s) {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n\ts_setprio 0" ::: "memory");
    const int kb = 2 * s + grp;
    if (kb >= KB) continue;   // wave-uniform
    const uint8_t *st = gs + (s & 1) * C::kStageBytes;
    if (kb + 2 < KB) issue(kb + 2, gs + ((s + 1) & 1) * C::kStageBytes);
    BlockScales cur;
    read_scales(kb, st, cur);
    v8i af[4], bf[4];
    af[0] = frag(st, wm + (lane & 15), lane);
    bf[0] = frag(st + C::kABytes, wn + (lane & 15), lane);
    bf[1] = frag(st + C::kABytes, wn + 16 + (lane & 15), lane);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q < 2) bf[q + 2] = frag(st + C::kABytes, wn + 16 * (q + 2) + (lane & 15), lane);
      else if (q < 5) af[q - 1] = frag(st, wm + 16 * (q - 1) + (lane & 15), lane);
      const int mi = q >> 2, ni = (mi & 1) ? 3 - (q & 3) : (q & 3), i = 4 * mi + ni;
      promote(acc[i], p[i], prev, mi);
      p[i] = mfma_k128(bf[ni], af[mi]);
      if (q == 0) __builtin_amdgcn_s_setprio(3);
      __builtin_amdgcn_sched_barrier(0);
    }
    prev = cur;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) promote(acc[i], p[i], prev, i >> 2);

  // group 1 -> LDS (every stage read is done once all waves pass this barrier)
  asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  v4f *red = reinterpret_cast<v4f *>(smem) + wv * 16 * 64 + lane;
  if (grp == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[i * 64] = acc[i];
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (grp == 1) return;
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int64_t i = m0 + wm + 16 * mi + (lane & 15);
    if (i >= m) continue;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t j = n0 + wn + 16 * ni + 4 * (lane >> 4);
      if (j >= n) continue;
      const v4f a = acc[4 * mi + ni] + red[(4 * mi + ni) * 64];
      store_bf16x4(reinterpret_cast<uint16_t *>(g.D) + i * g.ldd + j, a, n - j);
    }
  }
}

// UE8M0 group-32 recipe: both operands carry one power-of-two scale per row and
// 32-wide K group (packed as in "deep-gemm: fused per-token FP8 cast in Triton":
// the word of 128-K block kb holds the exponent bytes e+127 of its four groups).
// V_MFMA_SCALE_F32_16X16X128_F8F6F4 takes one E8M0 scale per lane, and (measured
// on MI355X) the scale of lane l covers row l&15 in register half (l>>5) (v0-3
// or v4-7) of lane groups 2((l>>4)&1) and 2((l>>4)&1)+1.  Loading a lane of group
// G = l>>4 with the row's 16-byte chunks G (into v0-3) and G+4 (into v4-7) --
// the same K order for both operands -- puts 32-K group G of the block exactly
// under the scale of lanes 16G..16G+15, which is byte G of the packed word.  The
// scaling then happens inside the MFMA, which accumulates straight into the
// fp32 accumulator: no promotion.  Each register half holds 16 consecutive
// K bytes, so the MFMA's runs of 8 products are still 8 consecutive K.  Tiles,
// copies, waits and fragment order are those of gemm_kernel.  (The weight
// gradients with these scales run on gemm_wgrad_kernel, for its precision.)
__device__ __forceinline__ v8i frag_g32(const uint8_t *tile, int row, int lane) {
  const int c = lane >> 4;
  const u32x4 lo = *reinterpret_cast<const u32x4 *>(tile + swz(row, c));
  const u32x4 hi = *reinterpret_cast<const u32x4 *>(tile + swz(row, c + 4));
  v8i r;
  r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
  r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
  return r;
}

// Exponent layouts of the scaled-MFMA kernel: kUeG32Packed, one word per row and
// 128-K block holding its four 32-K groups' bytes; kUeG128Packed, one word per row
// and four 128-K blocks (byte kb%4 of word kb/4); kUeG128Float, one fp32 2^e per
// row and 128-K block (the UE8M0 per-token cast), whose bits 30-23 are e+127.
// kUeBlockFloat (B only): one fp32 2^e per 128x128 block of B, (nb, kb) at
// sb[nb*sb_ld + kb], the same exponent for every column of the tile.
enum : int { kUeG32Packed = 0, kUeG128Packed = 1, kUeG128Float = 2, kUeBlockFloat = 3 };

template <class C, bool GROUPED, int SMODE = kUeG32Packed, int SB_MODE = SMODE>
__global__ __launch_bounds__(C::kThreads, C::kMinBlocks) void gemm_g32_kernel(GemmArgs g, int tiles_m, int tiles_n) {
  // the stages, then a 1 KB slot that receives the B prefetch copies
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kStages * C::kStageBytes + 1024];
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = (wv / C::WAVES_N_) * 64, wn = (wv % C::WAVES_N_) * 64;
  int64_t m0, n0;
  if (!tile_origin<C>(tiles_m, tiles_n, m0, n0)) return;
  const int64_t m = g.m, n = g.n;
  const int KB = (int)(g.k / kBK);

  // m-grouped layout (as in gemm_kernel): the tile's rows belong to the expert with
  // the largest m_indices among them; a tile without a valid expert returns whole.
  const uint8_t *Bg = g.B;
  const uint32_t *sbw = reinterpret_cast<const uint32_t *>(g.sb);
  int expert = 0;
  if constexpr (GROUPED) {
    static_assert(C::kBM == 128, "one 128-row segment block per tile");
    uint32_t v = 0;
#pragma unroll
    for (int r = 0; r < C::kBM; r += 64)
      if (m0 + r + lane < m) v = max(v, (uint32_t)(g.m_idx[m0 + r + lane] + 1));
    expert = (int)wave_max_u32(v) - 1;
    if (expert < 0 || expert >= g.num_experts) return;
    Bg = g.B + (int64_t)expert * g.b_estride;
    sbw += (int64_t)expert * g.sb_estride;
  }

  // one stage: the A and B tiles of K block kb and the scale words of the tile's
  // rows (A) and columns (B), or B's one block scale
  const TileCopy<C> cp(g, m0, n0, wv, lane);
  const uint32_t *saw = reinterpret_cast<const uint32_t *>(g.sa);
  auto issue = [&](int kb, uint8_t *st) {
    cp.tiles(g.A + m0 * g.lda + (int64_t)kb * kBK, Bg + n0 * g.ldb + (int64_t)kb * kBK, st, wv);
    const int64_t col_a = SMODE == kUeG128Packed ? (kb >> 2) : kb;
    const int64_t col_b = SB_MODE == kUeG128Packed ? (kb >> 2) : kb;
    const uint32_t *sb_row = SB_MODE == kUeBlockFloat ? sbw + (n0 >> 7) * g.sb_ld + kb : sbw + col_b * g.sb_ld + n0;
    cp.scales(saw + col_a * g.sa_ld + m0, sb_row, SB_MODE == kUeBlockFloat, st, wv);
  };

  v4f acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  // this lane's 32-K group within the block (group 32), the fp32 exponent field, or
  // (packed group 128, below) the block's byte of its word
  auto shift0 = [&](int mode) { return mode == kUeG32Packed ? 8 * (lane >> 4) : mode == kUeG128Packed ? 0 : 23; };
  const int gsh_a0 = shift0(SMODE), gsh_b0 = shift0(SB_MODE);
  issue(0, smem);
  // B prefetch of the first round of workgroups, as in gemm_kernel
  const bool prefetching = !GROUPED && (int)blockIdx.x < g.b_prefetch_wgs;
  if (prefetching) b_prefetch<C>(g, n, wv, lane, smem + C::kStages * C::kStageBytes);
  for (int kb = 0; kb < KB; ++kb) {
    if (prefetching && kb == 0)   // block 0 has landed; the prefetch copies may be in flight
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n\ts_setprio 0" ::"n"(kPrefetch) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n\ts_setprio 0" ::: "memory");
    const uint8_t *st = smem + (kb & 1) * C::kStageBytes;
    if (kb + 1 < KB) issue(kb + 1, smem + ((kb + 1) & 1) * C::kStageBytes);
    const int gsh_a = SMODE == kUeG128Packed ? 8 * (kb & 3) : gsh_a0;
    const int gsh_b = SB_MODE == kUeG128Packed ? 8 * (kb & 3) : gsh_b0;
    int ea[4], eb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ea[i] = (int)((*reinterpret_cast<const uint32_t *>(st + C::kSaOff + 4 * (wm + 16 * i + (lane & 15))) >> gsh_a) &
                    0xFFu);
      const int bo = SB_MODE == kUeBlockFloat ? 0 : 4 * (wn + 16 * i + (lane & 15));
      eb[i] = (int)((*reinterpret_cast<const uint32_t *>(st + C::kSbOff + bo) >> gsh_b) & 0xFFu);
    }
    v8i af[4], bf[4];
    af[0] = frag_g32(st, wm + (lane & 15), lane);
    bf[0] = frag_g32(st + C::kABytes, wn + (lane & 15), lane);
    bf[1] = frag_g32(st + C::kABytes, wn + 16 + (lane & 15), lane);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q < 2) bf[q + 2] = frag_g32(st + C::kABytes, wn + 16 * (q + 2) + (lane & 15), lane);
      else if (q < 5) af[q - 1] = frag_g32(st, wm + 16 * (q - 1) + (lane & 15), lane);
      const int mi = q >> 2, ni = (mi & 1) ? 3 - (q & 3) : (q & 3), i = 4 * mi + ni;
      // first operand B (its lane's column scale), second A (its lane's row scale)
      acc[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[ni], af[mi], acc[i], 0, 0, 0, eb[ni], 0, ea[mi]);
      if (q == 0) __builtin_amdgcn_s_setprio(3);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int64_t i = m0 + wm + 16 * mi + (lane & 15);
    if (i >= m) continue;
    if constexpr (GROUPED) {
      if (g.m_idx[i] != expert) continue;   // padding (or another expert's) row
    }
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
      const int64_t j = n0 + wn + 16 * ni + 4 * (lane >> 4);
      if (j >= n) continue;
      const v4f a = acc[4 * mi + ni];
      uint16_t *dp = reinterpret_cast<uint16_t *>(g.D) + i * g.ldd + j;
      if (j + 4 <= n) {
        *reinterpret_cast<u32x2 *>(dp) = (u32x2){bf16_rne(a[0]) | (bf16_rne(a[1]) << 16),
                                                 bf16_rne(a[2]) | (bf16_rne(a[3]) << 16)};
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (j + r < n) dp[r] = (uint16_t)bf16_rne(a[r]);
      }
    }
  }
}

// Weight gradient ("DeepGEMM Essentials", Parts 12-13: K runs over tokens, both
// operands carry one scale per row and 128-token block -- or, in the UE8M0
// recipes, a power of two per row and 128- or 32-token group -- and the fp32
// output is accumulated in place) on the bf16 MFMA.
//
// Why not the FP8 MFMA: it adds each run of 8 consecutive K products after
// aligning them to the run's largest exponent sum with 13 fraction bits,
// truncated, which on randn operands leaves a relative Frobenius error of
// 1.35e-5 (fp32 scales) to 1.5e-5 (UE8M0 scales) in a 4096 x 7168 gradient over
// 8192 tokens, above the 1e-5 the gradient must meet.  V_MFMA_F32_16X16X32_BF16
// (and _F16) sum a 128-wide K block to within ~1e-8 (measured on MI355X), and
// every E4M3 value is exact in bf16, also after a power-of-two scale, so this
// kernel keeps gemm_kernel's FP8 tiles, copies and pipeline and widens the
// fragments in registers just before the MFMAs (V_CVT_SCALEF32_PK_BF16_FP8:
// exact for all 256 codes).  A lane's 32 K bytes of a fragment row are read 16
// at a time; 8-byte slice s feeds the block's s-th MFMA, in the same order for
// both operands, so the four MFMAs of a tile add all 128 products of the block.
// With fp32 scales they go into a fresh partial sum P, promoted with
// sa(i, kb) * sb(j, kb) in the block's last slice, each tile four MFMAs after its
// last one.  (bf16 rather than f16: the same sums, and the bf16 MFMA measured
// 2-10% faster in this kernel on MI355X.)
//
// Cost, measured on MI355X: with two waves per SIMD a conversion costs about as
// much issue time as an FMA, and VALU instructions beyond the first one or two per
// MFMA add their issue time to the MFMA's, so with two conversions and two
// promotion instructions per 16x16x32 MFMA the fp32-scale kernel is bound by VALU
// issue (MFMA busy ~46% of cycles): 430-490 us for 4096 x 7168 x 8192, 326 us with
// the VALU work removed in a timing-only build; UE8M0 scales (no promotion)
// 389-402 us; the same pipeline on the FP8 MFMA 305-311 us.
typedef __bf16 b8 __attribute__((ext_vector_type(8)));

// bf16 operand of slice s of 16 FP8 bytes, each value times the power of two
// `scale` (exact: E4M3 has 4 significant bits, bf16 8, and the exponent range of
// fp32)
__device__ __forceinline__ b8 slice_bf16(const u32x4 &raw, int s, float scale) {
  const uint32_t w0 = raw[2 * s], w1 = raw[2 * s + 1];
  const u32x4 d = {__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, scale, true)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, false)),
                   __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, scale, true))};
  return __builtin_bit_cast(b8, d);
}

// Scale layouts of the weight-gradient kernel: kWgFp32, one fp32 scale per row and
// 128-K block (promoted); the UE8M0 layouts of gemm_g32_kernel (kUeG32Packed,
// kUeG128Packed, kUeG128Float) on both operands, folded into the conversion.
constexpr int kWgFp32 = -1;

// Weight-gradient kernel.  SMODE == kWgFp32: fragments widened to bf16 (scale 1),
// the block's partial sums promoted with sa(i, kb) * sb(j, kb).  UE8M0 layouts:
// each fragment widened to bf16 times its row's power of two for the lane's
// 32-K group (the lane of group G = lane/16 holds K bytes 32G..32G+31 of the
// block, so with 1x32 groups that is byte G of the block's word), and the MFMAs
// accumulate straight into the output registers over all of K: no promotion.
template <class C, int SMODE>
__global__ __launch_bounds__(C::kThreads, C::kMinBlocks) void gemm_wgrad_kernel(GemmArgs g, int tiles_m,
                                                                               int tiles_n) {
  static_assert(C::kBM == 128 && C::kBN == 128 && C::kStages == 2, "128x128 tiles, two stages");
  constexpr bool kUe = SMODE != kWgFp32;
  // the stages, then a 1 KB slot that receives the D prefetch copies
  __shared__ __attribute__((aligned(1024))) uint8_t smem[C::kStages * C::kStageBytes + 1024];
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = (wv / C::WAVES_N_) * 64, wn = (wv % C::WAVES_N_) * 64;
  int64_t m0, n0;
  if (!tile_origin<C>(tiles_m, tiles_n, m0, n0)) return;
  const int KB = (int)(g.k / kBK);

  // one stage: the A and B tiles of K block kb, sa's rows and sb's columns (MN-major;
  // packed 1x128 words hold four K blocks)
  const TileCopy<C> cp(g, m0, n0, wv, lane);
  const uint32_t *saw = reinterpret_cast<const uint32_t *>(g.sa);
  const uint32_t *sbw = reinterpret_cast<const uint32_t *>(g.sb);
  auto issue = [&](int kb, uint8_t *st) {
    cp.tiles(g.A + m0 * g.lda + (int64_t)kb * kBK, g.B + n0 * g.ldb + (int64_t)kb * kBK, st, wv);
    const int64_t col = SMODE == kUeG128Packed ? (kb >> 2) : kb;
    cp.scales(saw + col * g.sa_ld + m0, sbw + col * g.sb_ld + n0, false, st, wv);
  };

  v4f acc[16], p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  // Two stages, waits and wave priorities as in gemm_kernel.  D is read at the
  // end, written a whole step earlier: the tile's D is pulled into the caches
  // behind block 0's copies (d_prefetch).
  issue(0, smem);
  const bool prefetching = d_prefetch<C>(g, m0, n0, wv, lane, smem + C::kStages * C::kStageBytes);
  for (int kb = 0; kb < KB; ++kb) {
    if (prefetching && kb == 0)   // block 0 has landed; the prefetch copies may be in flight
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n\ts_setprio 0" ::"n"(kPrefetch) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier\n\ts_setprio 0" ::: "memory");
    const uint8_t *st = smem + (kb & 1) * C::kStageBytes;
    if (kb + 1 < KB) issue(kb + 1, smem + ((kb + 1) & 1) * C::kStageBytes);
    // UE8M0: the lane's powers of two for this block (row-subtile i of A, of B)
    float ea[4], eb[4];
    if constexpr (kUe) {
      const int sh = SMODE == kUeG32Packed ? 8 * (lane >> 4) : SMODE == kUeG128Packed ? 8 * (kb & 3) : 23;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t wa = *reinterpret_cast<const uint32_t *>(st + C::kSaOff + 4 * (wm + 16 * i + (lane & 15)));
        const uint32_t wb = *reinterpret_cast<const uint32_t *>(st + C::kSbOff + 4 * (wn + 16 * i + (lane & 15)));
        ea[i] = __uint_as_float(((wa >> sh) & 0xFFu) << 23);
        eb[i] = __uint_as_float(((wb >> sh) & 0xFFu) << 23);
      }
    }
    // fp32: row scale of each row-subtile and the 4 column scales of each
    // column-subtile, read from the stage (intact until block kb+2's copies) in
    // the last slice, where the promotion uses them
    float sa[4];
    v4f sbj[4];
    // tile at snake position q (row 0 left to right, row 1 right to left, ...)
    auto tile = [](int q, int &mi, int &ni) {
      mi = q >> 2;
      ni = (mi & 1) ? 3 - (q & 3) : (q & 3);
    };
    auto promote_tile = [&](int q) {
      int mi, ni;
      tile(q, mi, ni);
      const int i = 4 * mi + ni;
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][r] = __builtin_fmaf(p[i][r], sa[mi] * sbj[ni][r], acc[i][r]);
    };
    // 16 K bytes of each fragment row per half h: slices 2h and 2h + 1 (both halves
    // read at the block's start, so the second half's reads overlap the first's MFMAs)
    u32x4 af2[2][4], bf2[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 2 * (lane >> 4) + h;   // the frag() layout's chunk of this half
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af2[h][i] = *reinterpret_cast<const u32x4 *>(st + swz(wm + 16 * i + (lane & 15), c));
        bf2[h][i] = *reinterpret_cast<const u32x4 *>(st + C::kABytes + swz(wn + 16 * i + (lane & 15), c));
      }
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const u32x4 *af = af2[s >> 1], *bf = bf2[s >> 1];
      if constexpr (kUe) {
        b8 ah[4], bh[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ah[i] = slice_bf16(af[i], s & 1, ea[i]);
          bh[i] = slice_bf16(bf[i], s & 1, eb[i]);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          int mi, ni;
          tile(q, mi, ni);
          const int i = 4 * mi + ni;
          acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[ni], ah[mi], acc[i], 0, 0, 0);
          if (s == 0 && q == 0) __builtin_amdgcn_s_setprio(3);
        }
      } else {
        if (s == 3) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sa[i] = *reinterpret_cast<const float *>(st + C::kSaOff + 4 * (wm + 16 * i + (lane & 15)));
            sbj[i] = *reinterpret_cast<const v4f *>(st + C::kSbOff + 4 * (wn + 16 * i + 4 * (lane >> 4)));
          }
        }
        b8 ah[4], bh[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ah[i] = slice_bf16(af[i], s & 1, 1.0f);
          bh[i] = slice_bf16(bf[i], s & 1, 1.0f);
        }
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          int mi, ni;
          tile(q, mi, ni);
          const int i = 4 * mi + ni;
          const v4f c = s == 0 ? (v4f){0.0f, 0.0f, 0.0f, 0.0f} : p[i];
          p[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh[ni], ah[mi], c, 0, 0, 0);
          if (s == 0 && q == 0) __builtin_amdgcn_s_setprio(3);
          if (s == 3 && q >= 4) promote_tile(q - 4);
        }
      }
    }
    if constexpr (!kUe) {
#pragma unroll
      for (int q = 12; q < 16; ++q) promote_tile(q);
    }
  }
  wgrad_store(g, acc, m0, n0, wm, wn, lane);
}

// Skinny (decode-sized) problems, m <= 16*MT: there is too little output to fill
// 256 CUs with 128x128 tiles (m = 1, n = 7168 gives 56 tiles), and the time goes
// into streaming B once from HBM.  A workgroup owns 16*NT columns (inside one
// 128-column block, so one RHS block scale per K block) and all 16*MT rows; its W
// waves take the K blocks round-robin (wave w: blocks w, w + W, ...), load their
// fragments straight into VGPRs through a DEPTH-deep register ring (no LDS
// staging: nothing is reused across waves) and keep their own promoted fp32
// accumulators.  The W partial accumulators are then added through LDS in wave
// order, so the result does not depend on scheduling.
template <int MT, int NT, int W, int DEPTH, int SA_FMT>
__global__ __launch_bounds__(64 * W) void gemm_skinny_kernel(GemmArgs g, int tiles_n) {
  static_assert(128 % (16 * NT) == 0, "a workgroup's columns lie in one 128-column block");
  __shared__ v4f red[W][MT * NT][64];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tn = (int)(blockIdx.x % tiles_n), tm = (int)(blockIdx.x / tiles_n);
  const int64_t m0 = (int64_t)tm * 16 * MT, n0 = (int64_t)tn * 16 * NT;
  const int64_t m = g.m, n = g.n;
  const int KB = (int)(g.k / kBK);
  const int koff = 32 * (lane >> 4);   // this lane's K bytes within a block (frag() layout)

  const uint8_t *pa[MT];
  bool va[MT];
  int64_t ra[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t row = m0 + 16 * t + (lane & 15);
    va[t] = row < m;
    ra[t] = min(row, m - 1);
    pa[t] = g.A + ra[t] * g.lda + koff;
  }
  const uint8_t *pb[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) pb[t] = g.B + min(n0 + 16 * t + (lane & 15), n - 1) * g.ldb + koff;
  const float *psb = g.sb + (n0 >> 7) * g.sb_ld;

  struct Blk {
    v8i a[MT], b[NT];
    float sa[MT], sb;
  };
  auto load = [&](int kb, Blk &x) {
    const int64_t o = (int64_t)kb * kBK;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const u32x4 lo = *reinterpret_cast<const u32x4 *>(pb[t] + o);
      const u32x4 hi = *reinterpret_cast<const u32x4 *>(pb[t] + o + 16);
      x.b[t] = (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      x.a[t] = (v8i){0, 0, 0, 0, 0, 0, 0, 0};
      if (va[t]) {
        const u32x4 lo = *reinterpret_cast<const u32x4 *>(pa[t] + o);
        const u32x4 hi = *reinterpret_cast<const u32x4 *>(pa[t] + o + 16);
        x.a[t] = (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
      }
      x.sa[t] = load_sa<SA_FMT>(g.sa, g.sa_ld, ra[t], kb);
    }
    x.sb = psb[kb];
  };

  v4f acc[MT * NT];
#pragma unroll
  for (int i = 0; i < MT * NT; ++i) acc[i] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  auto compute = [&](const Blk &x) {
#pragma unroll
    for (int tm_ = 0; tm_ < MT; ++tm_) {
      const float c = x.sa[tm_] * x.sb;
#pragma unroll
      for (int tn_ = 0; tn_ < NT; ++tn_) {
        const v4f p = mfma_k128(x.b[tn_], x.a[tm_]);
        v4f &a = acc[tm_ * NT + tn_];
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = __builtin_fmaf(p[r], c, a[r]);
      }
    }
  };

  // Register ring: block j of this wave (kb = wv + j*W) lives in buf[j % DEPTH];
  // loads run DEPTH - 1 blocks ahead of the MFMAs.
  const int nblk = wv < KB ? (KB - 1 - wv) / W + 1 : 0;
  Blk buf[DEPTH];
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d)
    if (d < nblk) load(wv + d * W, buf[d]);
  for (int j0 = 0; j0 < nblk; j0 += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int j = j0 + d;
      if (j < nblk) {
        const int jn = j + DEPTH - 1;
        if (jn < nblk) load(wv + jn * W, buf[(d + DEPTH - 1) % DEPTH]);
        compute(buf[d]);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < MT * NT; ++i) red[wv][i][lane] = acc[i];
  __syncthreads();
  for (int i = wv; i < MT * NT; i += W) {
    v4f sum = red[0][i][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += red[w][i][lane];
    const int64_t row = m0 + 16 * (i / NT) + (lane & 15);
    const int64_t col = n0 + 16 * (i % NT) + 4 * (lane >> 4);
    if (row >= m || col >= n) continue;
    uint16_t *dp = reinterpret_cast<uint16_t *>(g.D) + row * g.ldd + col;
    if (col + 4 <= n) {
      *reinterpret_cast<u32x2 *>(dp) = (u32x2){bf16_rne(sum[0]) | (bf16_rne(sum[1]) << 16),
                                               bf16_rne(sum[2]) | (bf16_rne(sum[3]) << 16)};
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (col + r < n) dp[r] = (uint16_t)bf16_rne(sum[r]);
    }
  }
}

// Wait until at most n (0 <= n < 32) vector memory operations of this wave are
// outstanding, then meet the other waves at the barrier.  The count must be an
// immediate: with n known at compile time (an unrolled loop) the chain folds to one
// instruction pair.
template <int N = 0>
__device__ __forceinline__ void vm_wait_barrier(int n) {
  if constexpr (N < 32) {
    if (n == N) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
      return;
    }
    vm_wait_barrier<N + 1>(n);
  } else {
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  }
}

// Stream-K decode GEMM (m <= 16*MT <= 64), bf16 output.  The K blocks of all
// 128-column tiles form one list of units (tile-major, a tile's KB = k/128 blocks
// in order); workgroup w takes units [w*UPW, w*UPW + UPW), so the work splits into
// equal shares whatever the tile count, and a share may end inside one tile and
// start the next.  A workgroup of 8 waves issues every copy of its share at once:
// A's rows of each unit into LDS (the swizzled layout and direct-to-LDS copies of
// gemm_kernel, one 1 KB copy per wave per unit), each wave's 16 columns of B
// straight into registers; then it takes the units in order as they land, one FP8
// MFMA per 16-row subtile and the fp32 promotion by sa(i, kb) * sb(tile, kb).
//
// A tile that one workgroup covers whole is rounded and stored directly.  A tile
// shared by consecutive workgroups gets each sharer's fp32 partial sum in the
// workspace (slot 2w for the tile a share starts in, 2w+1 for the one it ends in;
// a slot holds the 16*MT x 128 fp32 in the order the waves hold them, [wave][row
// subtile][lane][4], so each store is 1 KB contiguous), and streamk_fixup_kernel
// adds them in workgroup order next.
template <int MT, int UPW, int SA_FMT>
__global__ __launch_bounds__(512) void gemm_streamk_kernel(GemmArgs g, float *part, int units) {
  constexpr int R = 16 * MT;     // A rows staged (rows past m repeat row m-1)
  constexpr int kCopies = R / 8; // 1 KB copies per unit (8 rows each)
  __shared__ __attribute__((aligned(1024))) uint8_t atile[UPW * R * kBK];
  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t m = g.m, n = g.n;
  const int KB = (int)(g.k / kBK);
  const int w = (int)blockIdx.x, u0 = w * UPW, nu = min(UPW, units - u0);   // nu >= 1 (host plan)
  const int t0 = u0 / KB;

  // per unit j (units past the share repeat its last one): tile, K block, scales
  int ut[UPW], ukb[UPW];
  float sa[UPW][MT], sb[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int u = u0 + min(j, nu - 1);
    ut[j] = u / KB;
    ukb[j] = u - ut[j] * KB;
    sb[j] = g.sb[(int64_t)ut[j] * g.sb_ld + ukb[j]];
#pragma unroll
    for (int i = 0; i < MT; ++i)
      sa[j][i] = load_sa<SA_FMT>(g.sa, g.sa_ld, min((int64_t)(16 * i + (lane & 15)), m - 1), ukb[j]);
  }
  // A of every unit -> LDS: wave wv fills copy wv % kCopies of each unit (slot s of a
  // copy: row s/8 of its 8, physical chunk s%8 holding logical chunk (s%8)^swz_key(row));
  // waves past kCopies repeat a copy, so each wave issues exactly UPW copies.
  {
    const int q = wv % kCopies, slot = 64 * q + lane;
    const int row = slot >> 3, chunk = (slot & 7) ^ swz_key(row);
    const uint32_t off = (uint32_t)(min((int64_t)row, m - 1) * g.lda) + (uint32_t)(chunk * 16);
#pragma unroll
    for (int j = 0; j < UPW; ++j) load_lds16(g.A + (int64_t)ukb[j] * kBK, off, atile + j * (R * kBK) + 1024 * q);
  }
  // B: this wave's 16 columns of each unit, 32 K bytes per lane (the frag() layout)
  v8i bfr[UPW];
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    const int64_t col = min((int64_t)ut[j] * 128 + 16 * wv + (lane & 15), n - 1);
    const uint8_t *pb = g.B + col * g.ldb + (int64_t)ukb[j] * kBK + 32 * (lane >> 4);
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(pb);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(pb + 16);
    bfr[j] = (v8i){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }

  v4f acc[MT], head[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  const int64_t ccol = 16 * wv + 4 * (lane >> 4);   // this lane's first column within a tile
  // sharers of tile t: the workgroups whose shares meet its units
  auto wlo_of = [&](int t) { return (int)((int64_t)t * KB / UPW); };
  auto whi_of = [&](int t) { return (int)(((int64_t)t * KB + KB - 1) / UPW); };
  bool has_head = false, stored = false;   // workgroup-uniform
#pragma unroll
  for (int j = 0; j < UPW; ++j) {
    // unit j's A copies have landed in every wave once each wave has at most the later
    // units' copies and all B loads outstanding (the compiler waits for bfr[j] itself);
    // after a store the count no longer holds, and the wait is for everything
    vm_wait_barrier(stored ? 0 : (UPW - 1 - j) + 2 * UPW);
    if (j >= nu) continue;   // workgroup-uniform
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const v4f p = mfma_k128(bfr[j], frag(atile + j * (R * kBK), 16 * i + (lane & 15), lane));
      const float c = sa[j][i] * sb[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][r] = __builtin_fmaf(p[r], c, acc[i][r]);
    }
    if (j == nu - 1 || ukb[j] != KB - 1) continue;   // the share's last segment stays in acc
    const int t = ut[j];
    if (wlo_of(t) == whi_of(t)) {
      // a whole tile: round and store
      uint16_t *dt = reinterpret_cast<uint16_t *>(g.D) + (int64_t)t * 128;
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const int64_t row = 16 * i + (lane & 15), col = (int64_t)t * 128 + ccol;
        if (row < m && col < n) store_bf16x4(dt + row * g.ldd + ccol, acc[i], n - col);
      }
      stored = true;
    } else {
      // the share's first tile, shared with earlier workgroups: its partial waits in head
#pragma unroll
      for (int i = 0; i < MT; ++i) head[i] = acc[i];
      has_head = true;
    }
#pragma unroll
    for (int i = 0; i < MT; ++i) acc[i] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  }

  // the share's last segment, tile t1: a whole tile, or shared
  const int t1 = (u0 + nu - 1) / KB;
  const bool tail_shared = wlo_of(t1) != whi_of(t1);
  if (!tail_shared) {
    uint16_t *dt = reinterpret_cast<uint16_t *>(g.D) + (int64_t)t1 * 128;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int64_t row = 16 * i + (lane & 15), col = (int64_t)t1 * 128 + ccol;
      if (row < m && col < n) store_bf16x4(dt + row * g.ldd + ccol, acc[i], n - col);
    }
  }
  if (!has_head && !tail_shared) return;   // workgroup-uniform

  // partial sums: slot 2w holds the share's first tile t0, slot 2w+1 its last tile when
  // that is another one
  constexpr int kSlot = 8 * MT * 64 * 4;   // floats
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (h == 0 ? !has_head : !tail_shared) continue;
    v4f *ps = reinterpret_cast<v4f *>(part + (int64_t)(h == 0 || t1 == t0 ? 2 * w : 2 * w + 1) * kSlot) +
              wv * MT * 64 + lane;
#pragma unroll
    for (int i = 0; i < MT; ++i) ps[i * 64] = h == 0 ? head[i] : acc[i];
  }
}

// D tile t (when shared) = bf16(sum of its sharers' partial sums in workgroup order).
// Workgroup (t, i) adds row subtile i: thread (wave v, lane l) the four columns that
// wave v's lane l held in gemm_streamk_kernel, eight sharers' loads in flight.
template <int MT>
__global__ __launch_bounds__(512) void streamk_fixup_kernel(GemmArgs g, const float *part, int upw) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int t = (int)blockIdx.x / MT, i = (int)blockIdx.x % MT;
  const int KB = (int)(g.k / kBK);
  const int wlo = (int)((int64_t)t * KB / upw), whi = (int)(((int64_t)t * KB + KB - 1) / upw);
  const int64_t row = 16 * i + (lane & 15), col = (int64_t)t * 128 + 16 * wv + 4 * (lane >> 4);
  if (wlo == whi || row >= g.m || col >= g.n) return;   // a whole tile is stored already
  constexpr int kSlot = 8 * MT * 64 * 4;
  const int64_t off = (int64_t)(wv * MT + i) * 64 + lane;   // v4f index within a slot
  v4f sum = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  for (int w0 = wlo; w0 <= whi; w0 += 8) {
    v4f v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int ww = min(w0 + q, whi);
      const int slot = (int)((int64_t)ww * upw / KB) == t ? 2 * ww : 2 * ww + 1;
      v[q] = reinterpret_cast<const v4f *>(part + (int64_t)slot * kSlot)[off];
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (w0 + q <= whi) sum += v[q];
  }
  store_bf16x4(reinterpret_cast<uint16_t *>(g.D) + row * g.ldd + col, sum, g.n - col);
}

// K-sliced 128x128 tiles: D = bf16 of the sum of the tile's S slot partials, added in
// slice order (deterministic).  One workgroup per (tile, wave quarter of the tile):
// thread t takes v4f positions t, t + 256, t + 512, t + 768 of that wave's 16 x 64
// lanes, with all S loads of a position issued before the adds.
template <class C, int S>
__global__ __launch_bounds__(256) void kslice_fixup_kernel(GemmArgs g, int tiles_n) {
  static_assert(C::kWaves == 4, "four 64x64 wave blocks per tile");
  const int tile = (int)blockIdx.x >> 2, wv = (int)blockIdx.x & 3;
  const int64_t m0 = (int64_t)(tile / tiles_n) * C::kBM, n0 = (int64_t)(tile % tiles_n) * C::kBN;
  const int wm = (wv / C::WAVES_N_) * 64, wn = (wv % C::WAVES_N_) * 64;
  const v4f *src = reinterpret_cast<const v4f *>(g.part) + ((int64_t)tile * S * C::kWaves + wv) * 1024;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int pos = r * 256 + (int)threadIdx.x, i = pos >> 6, lane = pos & 63;
    v4f v[S];
#pragma unroll
    for (int s = 0; s < S; ++s) v[s] = src[(int64_t)s * C::kWaves * 1024 + pos];
    v4f sum = v[0];
#pragma unroll
    for (int s = 1; s < S; ++s) sum += v[s];
    const int64_t row = m0 + wm + 16 * (i >> 2) + (lane & 15), col = n0 + wn + 16 * (i & 3) + 4 * (lane >> 4);
    if (row < g.m && col < g.n) store_bf16x4(reinterpret_cast<uint16_t *>(g.D) + row * g.ldd + col, sum, g.n - col);
  }
}

}  // namespace

// Compute units of the current device (queried once per device).
static int cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int c = cached[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) c = 256;
    cached[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

template <class C>
hipError_t launch_cfg(const GemmArgs &args, hipStream_t st) {
  const int tiles_m = (int)((args.m + C::kBM - 1) / C::kBM), tiles_n = (int)((args.n + C::kBN - 1) / C::kBN);
  const int tiles = tiles_m * tiles_n;
  const int per_xcd = (tiles + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds));
  GemmArgs a = args;
  // B prefetch for forward / dgrad grids of more than one round of tiles (not for
  // the weight gradient, whose B is twice as large and shared by fewer XCDs per
  // round: measured 1-3% slower with it on the FP8 MFMA, as is a one-round grid)
  const int64_t first_round = (int64_t)C::kMinBlocks * cu_count();
  a.b_prefetch_wgs = (!a.wgrad && grid.x > first_round) ? (int)first_round : 0;
#define FGFP8_GEMM(SAF, GR, CF) \
  hipLaunchKernelGGL((gemm_kernel<C, SAF, GR, CF>), grid, dim3(C::kThreads), 0, st, a, tiles_m, tiles_n)
  const bool packed = a.sa_fmt == kSfPackedUe8m0;
  if (a.wgrad) {
    hipLaunchKernelGGL((gemm_wgrad_kernel<C, kWgFp32>), grid, dim3(C::kThreads), 0, st, a, tiles_m, tiles_n);
  } else if (a.m_idx != nullptr || a.q != nullptr) {
    // the grouped layout and the fused output cast work on 128x128 tiles
    if constexpr (C::kBM == 128 && C::kBN == 128) {
      if (a.m_idx != nullptr) {
        if (packed) FGFP8_GEMM(kSfPackedUe8m0, true, 0); else FGFP8_GEMM(kSfFp32, true, 0);
      } else if (a.cq_fmt == kSfUe8m0) {
        if (packed) FGFP8_GEMM(kSfPackedUe8m0, false, 2); else FGFP8_GEMM(kSfFp32, false, 2);
      } else {
        if (packed) FGFP8_GEMM(kSfPackedUe8m0, false, 1); else FGFP8_GEMM(kSfFp32, false, 1);
      }
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    if (packed) FGFP8_GEMM(kSfPackedUe8m0, false, 0); else FGFP8_GEMM(kSfFp32, false, 0);
  }
#undef FGFP8_GEMM
  return hipGetLastError();
}

template <int MT, int NT, int W, int DEPTH>
hipError_t launch_skinny(const GemmArgs &a, hipStream_t st) {
  const int tiles_n = (int)((a.n + 16 * NT - 1) / (16 * NT));
  const int tiles_m = (int)((a.m + 16 * MT - 1) / (16 * MT));
  const dim3 grid((unsigned)(tiles_n * tiles_m));
  if (a.sa_fmt == kSfPackedUe8m0) {
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, NT, W, DEPTH, kSfPackedUe8m0>), grid, dim3(64 * W), 0, st, a, tiles_n);
  } else {
    hipLaunchKernelGGL((gemm_skinny_kernel<MT, NT, W, DEPTH, kSfFp32>), grid, dim3(64 * W), 0, st, a, tiles_n);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_g32(const GemmArgs &args, hipStream_t st) {
  using C = Cfg<2, 2, 2>;
  const int tiles_m = (int)((args.m + C::kBM - 1) / C::kBM), tiles_n = (int)((args.n + C::kBN - 1) / C::kBN);
  const int per_xcd = (tiles_m * tiles_n + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds));
  GemmArgs a = args;
  // weight gradient: UE8M0 scales folded into the bf16 conversion (no B prefetch,
  // as for the fp32-scale weight gradient)
  if (a.wgrad) {
    if (a.ue_gran == 32)
      hipLaunchKernelGGL((gemm_wgrad_kernel<C, kUeG32Packed>), grid, dim3(C::kThreads), 0, st, a, tiles_m, tiles_n);
    else if (a.sa_fmt == kSfPackedUe8m0)
      hipLaunchKernelGGL((gemm_wgrad_kernel<C, kUeG128Packed>), grid, dim3(C::kThreads), 0, st, a, tiles_m, tiles_n);
    else
      hipLaunchKernelGGL((gemm_wgrad_kernel<C, kUeG128Float>), grid, dim3(C::kThreads), 0, st, a, tiles_m, tiles_n);
    return hipGetLastError();
  }
  // B prefetch for grids of more than one round
  const int64_t first_round = (int64_t)C::kMinBlocks * cu_count();
  a.b_prefetch_wgs = grid.x > first_round ? (int)first_round : 0;
  if (a.ue_gran == 128)   // forward / dgrad with UE8M0 1x128 A scales and 128x128 B block scales
    if (a.sa_fmt == kSfPackedUe8m0)
      hipLaunchKernelGGL((gemm_g32_kernel<C, false, kUeG128Packed, kUeBlockFloat>), grid, dim3(C::kThreads), 0, st, a,
                         tiles_m, tiles_n);
    else
      hipLaunchKernelGGL((gemm_g32_kernel<C, false, kUeG128Float, kUeBlockFloat>), grid, dim3(C::kThreads), 0, st, a,
                         tiles_m, tiles_n);
  else if (a.m_idx != nullptr)
    hipLaunchKernelGGL((gemm_g32_kernel<C, true>), grid, dim3(C::kThreads), 0, st, a, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_g32_kernel<C, false>), grid, dim3(C::kThreads), 0, st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

static hipError_t launch_ksplit2(const GemmArgs &a, hipStream_t st) {
  using C = Cfg<2, 2, 2>;
  const int tiles_m = (int)((a.m + C::kBM - 1) / C::kBM), tiles_n = (int)((a.n + C::kBN - 1) / C::kBN);
  const int per_xcd = (tiles_m * tiles_n + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds));
  if (a.sa_fmt == kSfPackedUe8m0)
    hipLaunchKernelGGL((gemm_ksplit2_kernel<C, kSfPackedUe8m0>), grid, dim3(2 * C::kThreads), 0, st, a, tiles_m, tiles_n);
  else
    hipLaunchKernelGGL((gemm_ksplit2_kernel<C, kSfFp32>), grid, dim3(2 * C::kThreads), 0, st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs &a, hipStream_t st) {
  if (!a.wgrad && a.m_idx == nullptr && a.q == nullptr && a.m <= 64) {
    // decode-sized: stream B with K split over the waves of a workgroup
    if (a.m <= 16) return launch_skinny<1, 1, 8, 4>(a, st);
    // 16 waves (shorter K walk per wave) when the workgroups of 32 columns still
    // fit one per CU with 16 (or 32) rows each; else 8 waves over 32 (64) rows.
    // Measured on MI355X, m = 64, n = 4096, k = 7168: 16.5 us against 22.6 us.
    const int64_t wn = (a.n + 31) / 32, cus = cu_count();
    if ((a.m + 15) / 16 * wn <= cus) return launch_skinny<1, 2, 16, 2>(a, st);
    if ((a.m + 31) / 32 * wn <= cus) return launch_skinny<2, 2, 16, 2>(a, st);
    if (a.m <= 32) return launch_skinny<2, 2, 8, 2>(a, st);
    return launch_skinny<4, 2, 8, 2>(a, st);
  }
  // Fewer 128x128 tiles than CUs and a long K (m = 512 decode): two K chains per tile
  if (!a.wgrad && a.m_idx == nullptr && a.q == nullptr && a.k >= 8 * kBK &&
      ((a.m + 127) / 128) * ((a.n + 127) / 128) < cu_count())
    return launch_ksplit2(a, st);
  // 128x128 output tiles, 4 waves, 2 LDS stages (66 KB): two workgroups per CU, so
  // one workgroup's barrier and copy latency is covered by the other's MFMAs.
  return launch_cfg<Cfg<2, 2, 2>>(a, st);
}

constexpr int64_t kMaxSlices = 4;

// Split-K plans.  m > 64: 128x128 tiles, K cut into S slices, for at most 128 tiles
// (half the CUs of the 256-CU part: with more, the plain kernels already fill the
// part and the slices' extra pass over the partial sums loses).  S is the largest
// of 2..4 with at least 8 K blocks per slice, and at least 12 once tiles * S
// passes one workgroup per CU; S = 1 (the plain kernel, no workspace) when none
// qualifies.  Measured on MI355X (B streamed from HBM), plain -> sliced: 512 x
// 4096 x 7168 41 -> 33 us (S = 4), 128 x 4096 x 7168 41 -> 20 us, 256 x 7168 x
// 4096 26 -> 23 us (S = 2, where S = 4 took 26 us).  m <= 64 (stream-K): units = 128-column tiles x K blocks; UPW units per
// workgroup, the fewest (at most 8) that keep the workgroups within one per CU of
// the 256-CU part (more than 256 only when that takes over 8 units each).
SplitKPlan splitk_plan(int64_t m, int64_t n, int64_t k) {
  SplitKPlan p;
  p.tiles_n = (n + 127) / 128;
  if (m > 64) {
    p.tiles_m = (m + 127) / 128;
    const int64_t tiles = p.tiles_m * p.tiles_n;
    const int64_t kb = k / kBK;
    p.slices = 1;
    if (tiles <= kStreamKSlots / 2)
      for (int64_t s = kMaxSlices; s >= 2; --s)
        if (kb >= 8 * s && (tiles * s <= kStreamKSlots || kb >= 12 * s)) {
          p.slices = s;
          break;
        }
    p.units = p.upw = 0;
    p.grid = tiles * p.slices;
    p.workspace_bytes = p.slices > 1 ? tiles * p.slices * 128 * 128 * (int64_t)sizeof(float) : 0;
    return p;
  }
  p.units = p.tiles_n * (k / kBK);
  p.upw = std::min<int64_t>(8, std::max<int64_t>(1, (p.units + kStreamKSlots - 1) / kStreamKSlots));
  p.grid = (p.units + p.upw - 1) / p.upw;
  // two slots per workgroup of the 16*MT x 128 fp32 of a tile (MT = ceil(m/16), 1, 2 or 4)
  const int64_t rows = m <= 16 ? 16 : m <= 32 ? 32 : 64;
  p.workspace_bytes = 2 * p.grid * rows * 128 * (int64_t)sizeof(float);
  return p;
}

template <int MT, int UPW>
static void launch_streamk_cfg(const GemmArgs &a, float *part, const SplitKPlan &p, hipStream_t st) {
  const dim3 grid((unsigned)p.grid);
  if (a.sa_fmt == kSfPackedUe8m0)
    hipLaunchKernelGGL((gemm_streamk_kernel<MT, UPW, kSfPackedUe8m0>), grid, dim3(512), 0, st, a, part, (int)p.units);
  else
    hipLaunchKernelGGL((gemm_streamk_kernel<MT, UPW, kSfFp32>), grid, dim3(512), 0, st, a, part, (int)p.units);
}

template <int MT>
static void launch_streamk_mt(const GemmArgs &a, float *part, const SplitKPlan &p, hipStream_t st) {
  switch (p.upw) {
    case 1: launch_streamk_cfg<MT, 1>(a, part, p, st); break;
    case 2: launch_streamk_cfg<MT, 2>(a, part, p, st); break;
    case 3: launch_streamk_cfg<MT, 3>(a, part, p, st); break;
    case 4: launch_streamk_cfg<MT, 4>(a, part, p, st); break;
    case 5: launch_streamk_cfg<MT, 5>(a, part, p, st); break;
    case 6: launch_streamk_cfg<MT, 6>(a, part, p, st); break;
    case 7: launch_streamk_cfg<MT, 7>(a, part, p, st); break;
    default: launch_streamk_cfg<MT, 8>(a, part, p, st); break;
  }
  // shared tiles: one workgroup per row subtile; none is shared when every share holds
  // whole tiles (UPW a multiple of KB)
  if (p.upw % (a.k / kBK) != 0)
    hipLaunchKernelGGL(streamk_fixup_kernel<MT>, dim3((unsigned)(p.tiles_n * MT)), dim3(512), 0, st, a, part,
                       (int)p.upw);
}

static hipError_t launch_kslice(const GemmArgs &args, float *part, const SplitKPlan &p, hipStream_t st) {
  using C = Cfg<2, 2, 2>;
  const int tiles_m = (int)p.tiles_m, tiles_n = (int)p.tiles_n;
  const int per_xcd = (tiles_m * tiles_n + kXcds - 1) / kXcds;
  const dim3 grid((unsigned)(per_xcd * kXcds), (unsigned)p.slices);
  GemmArgs a = args;
  a.part = part;
  a.b_prefetch_wgs = 0;
  if (a.sa_fmt == kSfPackedUe8m0)
    hipLaunchKernelGGL((gemm_kernel<C, kSfPackedUe8m0, false, 0, true>), grid, dim3(C::kThreads), 0, st, a, tiles_m,
                       tiles_n);
  else
    hipLaunchKernelGGL((gemm_kernel<C, kSfFp32, false, 0, true>), grid, dim3(C::kThreads), 0, st, a, tiles_m, tiles_n);
  const dim3 fgrid((unsigned)(tiles_m * tiles_n * 4));
  switch (p.slices) {
    case 2: hipLaunchKernelGGL((kslice_fixup_kernel<C, 2>), fgrid, dim3(256), 0, st, a, tiles_n); break;
    case 3: hipLaunchKernelGGL((kslice_fixup_kernel<C, 3>), fgrid, dim3(256), 0, st, a, tiles_n); break;
    default: hipLaunchKernelGGL((kslice_fixup_kernel<C, 4>), fgrid, dim3(256), 0, st, a, tiles_n); break;
  }
  return hipGetLastError();
}

hipError_t launch_gemm_splitk(const GemmArgs &a, void *ws, const SplitKPlan &p, hipStream_t st) {
  float *part = static_cast<float *>(ws);
  if (a.m > 64) return p.slices > 1 ? launch_kslice(a, part, p, st) : launch_gemm(a, st);
  if (a.m <= 16) launch_streamk_mt<1>(a, part, p, st);
  else if (a.m <= 32) launch_streamk_mt<2>(a, part, p, st);
  else launch_streamk_mt<4>(a, part, p, st);
  return hipGetLastError();
}
}  // namespace fgfp8
