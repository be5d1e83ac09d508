// moe_device.h -- device helpers shared by libmoe's gfx950 kernels.
// Wave64 (CDNA4) throughout: every cross-lane step assumes 64 lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libmoe.h"

#define MOE_WAVE 64

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

namespace moe {

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16 with round-to-nearest-even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

// ---------------------------------------------------------------- softmax exp
// fp32 e^x for x in [-87, 0]: Cody & Waite argument reduction (Software
// Manual for the Elementary Functions, 1980), x = n ln2 + r with ln2 split
// as 355/512 plus a low correction; e^r from its degree-7 Taylor polynomial
// (coefficients 1/i! rounded from double) by Horner's rule with fused
// multiply-adds; times 2^n assembled in the exponent field. Every operation
// is written out so that no compiler contraction changes a rounding.
__device__ __forceinline__ float softmax_exp(float x) {
#pragma clang fp contract(off)
  const float kLog2e = 1.44269504088896341f;
  const float kLn2Hi = 0.693359375f;
  const float kLn2Lo = -2.12194440054690583e-4f;
  const float q7 = (float)(1.0 / 5040.0);
  const float q6 = (float)(1.0 / 720.0);
  const float q5 = (float)(1.0 / 120.0);
  const float q4 = (float)(1.0 / 24.0);
  const float q3 = (float)(1.0 / 6.0);
  float t = x * kLog2e;
  float n = __builtin_rintf(t);
  float r = __builtin_fmaf(-n, kLn2Hi, x);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = __builtin_fmaf(q7, r, q6);
  p = __builtin_fmaf(p, r, q5);
  p = __builtin_fmaf(p, r, q4);
  p = __builtin_fmaf(p, r, q3);
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  int ni = (int)n;
  float scale = __uint_as_float((uint32_t)(ni + 127) << 23);
  return p * scale;
}

// ---------------------------------------------------------------- noise
// SplitMix64 step (Steele, Lea & Flood, OOPSLA 2014) from state x.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// Approximate N(0,1) draw for (token t, expert e): Irwin-Hall sum of twelve
// 24-bit uniforms taken from SplitMix64 on counters (t*E+e)*12 + i, minus 6.
// The integer sum is exact, so the value is the same on any device.
__device__ __forceinline__ float noise_normal(uint64_t seed, uint32_t t, uint32_t e,
                                              uint32_t E) {
  uint64_t c = (uint64_t)t * E + e;
  int64_t s = 0;
#pragma unroll
  for (int i = 0; i < 12; ++i) s += (int64_t)(splitmix64(seed ^ (c * 12ull + i)) >> 40);
  return (float)((double)(s - 6ll * 16777216ll) * (1.0 / 16777216.0));
}

// ---------------------------------------------------------------- wave ops
// Butterfly over the 64 lanes (call with every lane active): level o
// combines lane i with lane i ^ o, o = 32, 16, 8, 4, 2, 1, without the LDS
// crossbar. gfx950's permlane swaps hand every lane the pair of values
// (lane & ~o, lane | o) for o = 32 and 16; inside a row of 16 lanes a
// rotation by 8 is xor 8, and after that level lanes i and i ^ 8 hold equal
// values, so the rotation by 4 (lane i receives lane i - 4 mod 16) brings
// the value of lane i ^ 4; quad permutations give xor 2 and xor 1. Each
// level applies op to the lane's own value and its partner's (at o = 32
// and 16 in lane order, which a commutative op does not see).
namespace detail {
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
}  // namespace detail

template <typename Op>
__device__ __forceinline__ uint32_t wave_butterfly(uint32_t v, Op op) {
  const auto p32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = op(p32[0], p32[1]);
  const auto p16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(p16[0], p16[1]);
  v = op(v, detail::dpp<0x128>(v));  // row_ror:8
  v = op(v, detail::dpp<0x124>(v));  // row_ror:4
  v = op(v, detail::dpp<0x4e>(v));   // quad_perm [2,3,0,1]
  v = op(v, detail::dpp<0xb1>(v));   // quad_perm [1,0,3,2]
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_butterfly(__float_as_uint(v), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  }));
}

// Sum over the wave pairing lane i with lane i^o for o = 32..1: lane 0's
// value is the halving tree a_i + a_{i+h}, h = 32, 16, ..., 1, and every
// lane ends with that same value (one rounded addition per level, and an
// addition does not depend on the order of its operands).
__device__ __forceinline__ float wave_tree_sum(float v) {
  return __uint_as_float(wave_butterfly(__float_as_uint(v), [](uint32_t a, uint32_t b) {
#pragma clang fp contract(off)
    const float r = __uint_as_float(a) + __uint_as_float(b);
    return __float_as_uint(r);
  }));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_butterfly(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

// 64-bit maximum: the largest high word, then the largest low word among
// the lanes that hold it.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32);
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? (uint32_t)v : 0u);
  return ((uint64_t)mh << 32) | ml;
}

// fp32 -> uint32 whose unsigned order is the float order (finite values).
__device__ __forceinline__ uint32_t orderable(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  uint32_t lane = __lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe

// ---------------------------------------------------------------- host side
namespace moe_host {
void set_error(const char* fmt, ...);
moe_status launch_status(const char* what);
inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }
}  // namespace moe_host
