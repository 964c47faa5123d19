// Device helpers shared by the gfx950 kernels of libscaled_fp8: format
// constants, the exponent-bias rule, the saturating FP8 cast, bf16 unpacking
// and max-reductions.  Written for CDNA4 (64-lane wavefronts) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/scaled_fp8.h"

namespace sfp8 {

typedef unsigned short us2 __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// OCP OFP8 constants.  E4M3: largest finite 448 = 1.75 * 2^8.  E5M2: largest
// finite 57344 = 1.75 * 2^15.  Both maxima have the float32 mantissa field
// 0x600000 (1.75), which the bias rule compares against.
// ---------------------------------------------------------------------------
template <int FMT> struct Fmt;
template <> struct Fmt<FP8_E4M3> {
  static constexpr float kMax = 448.0f;
  static constexpr int kEmax = 8;
};
template <> struct Fmt<FP8_E5M2> {
  static constexpr float kMax = 57344.0f;
  static constexpr int kEmax = 15;
};
constexpr uint32_t kMaxMantissaField = 0x600000u;   // 1.75 in float32 bits

__device__ __forceinline__ int fmt_emax(int fmt) { return fmt == FP8_E4M3 ? 8 : 15; }

// Exponent bias from |amax| given as float32 bits with the sign cleared:
//   bias = floor(log2(fmax / amax)) - margin, clamped to [lo, hi];
//   amax == 0, Inf or NaN -> 0.
// floor(log2(fmax/amax)) is emax - E - (m_amax > 1.75 ? 1 : 0), where
// amax = m_amax * 2^E with m_amax in [1, 2); subnormal amax is normalised
// with a count of leading zeros.  Pure integer arithmetic: exact.
// With `top_binade` the correction term is dropped (emax - E - margin): the
// OCP MX shared-exponent rule, which puts amax in the format's top binade
// and lets a significand above the format maximum's saturate.
__device__ __forceinline__ int bias_from_amax_bits(uint32_t abits, int emax, int margin,
                                                   int lo, int hi, bool top_binade = false) {
  abits &= 0x7fffffffu;
  if (abits == 0u || abits >= 0x7f800000u) return 0;
  int E;
  uint32_t mfield;
  const uint32_t efield = abits >> 23;
  if (efield == 0u) {
    const int p = 31 - __clz(abits);            // position of the leading one
    E = p - 149;
    mfield = (abits << (23 - p)) & 0x7fffffu;
  } else {
    E = (int)efield - 127;
    mfield = abits & 0x7fffffu;
  }
  int b = emax - E - (!top_binade && mfield > kMaxMantissaField ? 1 : 0) - margin;
  b = b < lo ? lo : b;
  b = b > hi ? hi : b;
  return b;
}

// 2^e as a float for e in [-126, 127] (normal numbers only).
__device__ __forceinline__ float pow2f(int e) {
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

// ---------------------------------------------------------------------------
// Saturating round-to-nearest-even cast of four floats to FP8, packed into
// one dword (element 0 in the low byte).  The explicit clamp makes the
// saturation independent of the conversion instruction's overflow handling;
// gfx950's v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 round to nearest even onto
// the OCP grids.  NaN lanes are patched by the caller from the input bits.
// ---------------------------------------------------------------------------
template <int FMT>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  constexpr float M = Fmt<FMT>::kMax;
  a = __builtin_amdgcn_fmed3f(a, -M, M);
  b = __builtin_amdgcn_fmed3f(b, -M, M);
  c = __builtin_amdgcn_fmed3f(c, -M, M);
  d = __builtin_amdgcn_fmed3f(d, -M, M);
  int w;
  if constexpr (FMT == FP8_E4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return (uint32_t)w;
}

template <int FMT>
__device__ __forceinline__ uint32_t cvt1(float a) {
  return cvt4<FMT>(a, 0.0f, 0.0f, 0.0f) & 0xffu;
}

// FP8 NaN code with the sign of a bf16 / f32 input.
__device__ __forceinline__ uint32_t nan_code_bf16(uint32_t h) { return 0x7fu | ((h >> 8) & 0x80u); }
__device__ __forceinline__ uint32_t nan_code_f32(uint32_t u) { return 0x7fu | ((u >> 24) & 0x80u); }

// bf16 pair in a dword -> floats (element 0 is the low half).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// |bf16| bits of both halves, packed max.
__device__ __forceinline__ us2 abs_bf16x2(uint32_t w) {
  return __builtin_bit_cast(us2, w & 0x7fff7fffu);
}
__device__ __forceinline__ us2 max_us2(us2 a, us2 b) { return __builtin_elementwise_max(a, b); }
__device__ __forceinline__ uint32_t hmax_us2(us2 a) { return a.x > a.y ? a.x : a.y; }

// ---------------------------------------------------------------------------
// Reductions of non-negative float bit patterns (as uint32, so that the
// order is the float order and NaN patterns sort above +Inf).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)v, off, kWave);
    v = v > o ? v : o;
  }
  return v;
}

// One atomicMax per workgroup into *out (float bits).  All threads of the
// block must call it; `red` is __shared__ scratch of blockDim/64 words.
__device__ __forceinline__ void block_max_to_global(uint32_t v, uint32_t* red, float* out) {
  v = wave_max_u32(v);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    const int nw = (blockDim.x + kWave - 1) / kWave;
    for (int i = 0; i < nw; ++i) m = m > red[i] ? m : red[i];
    if (m != 0u) atomicMax(reinterpret_cast<unsigned int*>(out), m);
  }
}

// One 64-bit atomicAdd per workgroup of the lanes' counts into *out, skipped
// when the workgroup's count is zero.  All threads of the block must call it;
// `red` is __shared__ scratch of blockDim/64 words (not shared with another
// reduction running in the same block).
__device__ __forceinline__ void block_sum_to_global(uint32_t v, uint32_t* red, unsigned long long* out) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += (uint32_t)__shfl_xor((int)v, off, kWave);
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  if (lane == 0) red[wid] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long s = 0;
    const int nw = (blockDim.x + kWave - 1) / kWave;
    for (int i = 0; i < nw; ++i) s += red[i];
    if (s != 0) atomicAdd(out, s);
  }
}

// Saturation count of four scaled values: those whose magnitude exceeds the
// format maximum (the cast clamps them to +-max; NaN compares false).
template <int FMT>
__device__ __forceinline__ uint32_t sat4(float a, float b, float c, float d) {
  constexpr float M = Fmt<FMT>::kMax;
  return (uint32_t)(__builtin_fabsf(a) > M) + (uint32_t)(__builtin_fabsf(b) > M) +
         (uint32_t)(__builtin_fabsf(c) > M) + (uint32_t)(__builtin_fabsf(d) > M);
}

// Max across aligned groups of 4 / 8 lanes (DPP quad permutes, half-row mirror).
__device__ __forceinline__ uint32_t group4_max(uint32_t v) {
  uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // lane ^ 1
  v = v > o ? v : o;
  o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);           // lane ^ 2
  return v > o ? v : o;
}
__device__ __forceinline__ uint32_t group8_max(uint32_t v) {
  v = group4_max(v);
  const uint32_t o = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);  // half-row mirror
  return v > o ? v : o;
}

}  // namespace sfp8
