// Shared device helpers of libcosa: storage types, conversions and MFMA wrappers
// for gfx950 (CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cosa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// bf16 is stored as its raw 16 bits.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// Round-to-nearest-even float -> bf16 (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// The same rounding (RNE) through gfx950's v_cvt_pk_bf16_f32: one instruction per pair.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Combine lane l with lane l ^ 32 via gfx950's v_permlane32_swap (no LDS traffic): with
// both operands equal, the swap leaves v[l % 32] in the first result and v[l % 32 + 32]
// in the second, on every lane, so both lanes of a pair get bitwise the same answer.
__device__ __forceinline__ float halves_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Element traits: how many elements one lane feeds a 32x32 MFMA per k-step.
template <typename T>
struct Mfma;

// v_mfma_f32_32x32x16_bf16: A 32x16, B 16x32, C 32x32 fp32.
// Lane l holds A[l%32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l%32];
// C element (row 8*i + 4*(l/32) + j, col l%32) sits in slot 4*i + j.
template <>
struct Mfma<bf16_t> {
  static constexpr int KSTEP = 16;  // k consumed per instruction
  static constexpr int KPL = 8;     // k elements per lane per instruction
  typedef bf16x8 frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

// v_mfma_f32_32x32x2_f32: A 32x2, B 2x32; lane l holds A[l%32][l/32], B[l/32][l%32].
template <>
struct Mfma<float> {
  static constexpr int KSTEP = 2;
  static constexpr int KPL = 1;
  typedef float frag;
  __device__ __forceinline__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Load KPL consecutive elements as an MFMA fragment (16 bytes for bf16, 4 for f32).
__device__ __forceinline__ bf16x8 load_frag(const bf16_t* p) {
  u32x4 v = *reinterpret_cast<const u32x4*>(p);
  return __builtin_bit_cast(bf16x8, v);
}
__device__ __forceinline__ float load_frag(const float* p) { return *p; }

__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x.bits); }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T>
__device__ __forceinline__ T from_f32(float f);
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) {
  bf16_t r;
  r.bits = f32_to_bf16(f);
  return r;
}
template <>
__device__ __forceinline__ float from_f32<float>(float f) {
  return f;
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

}  // namespace cosa
