// device_common.h -- small gfx950 device helpers shared by the cast and GEMM
// kernels of libfgfp8 (wave64 DPP reductions, E4M3 / bf16 rounding, the
// per-group scale rule).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fgfp8 {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// DPP lane exchanges inside a 16-lane row (no LDS traffic).
// ---------------------------------------------------------------------------
enum : int {
  kDppQuadXor1 = 0xB1,      // quad_perm [1,0,3,2]
  kDppQuadXor2 = 0x4E,      // quad_perm [2,3,0,1]
  kDppRowHalfMirror = 0x141,
  kDppRowMirror = 0x140,
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Max over groups of LANES consecutive lanes (LANES = 1, 2, 4, 8 or 16) of
// non-negative floats held as their bit patterns (integer order equals float
// order for non-negative values).
template <int LANES>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
  if constexpr (LANES >= 2) v = max(v, dpp<kDppQuadXor1>(v));
  if constexpr (LANES >= 4) v = max(v, dpp<kDppQuadXor2>(v));
  if constexpr (LANES >= 8) v = max(v, dpp<kDppRowHalfMirror>(v));
  if constexpr (LANES >= 16) v = max(v, dpp<kDppRowMirror>(v));
  return v;
}

// Bitwise OR over groups of LANES consecutive lanes (LANES <= 16).
template <int LANES>
__device__ __forceinline__ uint32_t group_or_u32(uint32_t v) {
  if constexpr (LANES >= 2) v |= dpp<kDppQuadXor1>(v);
  if constexpr (LANES >= 4) v |= dpp<kDppQuadXor2>(v);
  if constexpr (LANES >= 8) v |= dpp<kDppRowHalfMirror>(v);
  if constexpr (LANES >= 16) v |= dpp<kDppRowMirror>(v);
  return v;
}

// Max over the whole wave.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = group_max_u32<16>(v);
  uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

// ---------------------------------------------------------------------------
// Per-group scale.  amax is clamped at fp32(1e-4); the stored fp32 scale is
// amax/448 (IEEE division); the element multiplier is (1/amax)*448 with two
// roundings.  UE8M0: the least power of two 2^e >= amax/448, multiplier 2^-e.
// HIP compiles '/' on float to a correctly rounded division (no fast-math).
// ---------------------------------------------------------------------------
struct GroupScale {
  float sf;      // scale to store (fp32 or 2^e)
  float mult;    // multiplier for the group's elements
  uint32_t e8;   // e + 127 (UE8M0 formats only)
};

template <bool UE8M0>
__device__ __forceinline__ GroupScale group_scale(float amax) {
  const float kFloor = 1e-4f;
  GroupScale g;
  if (amax < kFloor) amax = kFloor;
  const float s = amax / 448.0f;
  if constexpr (!UE8M0) {
    const float recip = 1.0f / amax;
    g.sf = s;
    g.mult = recip * 448.0f;
    g.e8 = 0;
  } else {
    const uint32_t b = __float_as_uint(s);
    const uint32_t e8 = ((b >> 23) & 0xFFu) + ((b & 0x7FFFFFu) != 0u);   // biased exponent of 2^e
    g.e8 = e8;
    g.sf = __uint_as_float(e8 << 23);
    g.mult = __uint_as_float((254u - e8) << 23);                         // 2^-e
  }
  return g;
}

// ---------------------------------------------------------------------------
// E4M3 rounding of four fp32 values into one little-endian word, nearest
// with ties to even (the gfx950 OCP FP8 conversion).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// bf16 of an fp32 value, nearest with ties to even (finite inputs).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

}  // namespace fgfp8
