// Device-side helpers shared by the libmoe kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

typedef __bf16 bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define MOE_WAVE 64

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (round to nearest, ties to even; inputs here are finite)

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// gfx950 converts in hardware (v_cvt_pk_bf16_f32, round to nearest even)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ---------------------------------------------------------------------------
// Expert activation on the fp32 accumulators (g = gate projection,
// u = up projection). silu: g*sigmoid(g)*u. swigluoai: clamp g from above
// and u on both sides at `limit`, then g*sigmoid(alpha*g)*(u+beta).
//
// Both are one branch-free formula,
//   min(g, glimit) * sigmoid(alpha * min(g, glimit)) * (clamp(u, +-ulimit) + beta),
// with silu as the case glimit = ulimit = +inf, alpha = 1, beta = 0 (every
// step is then exact: min(g, inf) = g, 1*g = g, u + 0 = u), so the epilogues
// carry no per-element branch.

struct ActParams {
  float alpha, glimit, ulimit, beta;
};

// 1 / (1 + e^-z) with the hardware exp2 and reciprocal (about 1 ulp each);
// e^-z overflows to +inf for very negative z, and rcp(inf) = 0, as wanted.
__device__ __forceinline__ float sigmoid_f32(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ float act_apply(float g, float u, const ActParams& a) {
  const float gc = fminf(g, a.glimit);
  const float uc = fminf(fmaxf(u, -a.ulimit), a.ulimit);
  return gc * sigmoid_f32(a.alpha * gc) * (uc + a.beta);
}

// ---------------------------------------------------------------------------
// Eight consecutive elements of a row as fp32 (16-byte loads and stores of
// bf16, two of fp32); bf16 stores round to nearest even.

constexpr int VEC8 = 8;

template <typename T>
struct Vec8;
template <>
struct Vec8<float> {
  static __device__ __forceinline__ void load(const float* p, float (&v)[VEC8]) {
    const floatx4_t a = *reinterpret_cast<const floatx4_t*>(p);
    const floatx4_t b = *reinterpret_cast<const floatx4_t*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
  static __device__ __forceinline__ void store(float* p, const float (&v)[VEC8]) {
    *reinterpret_cast<floatx4_t*>(p) = floatx4_t{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<floatx4_t*>(p + 4) = floatx4_t{v[4], v[5], v[6], v[7]};
  }
};
template <>
struct Vec8<bf16_t> {
  static __device__ __forceinline__ void load(const bf16_t* p, float (&v)[VEC8]) {
    const u32x4_t u = *reinterpret_cast<const u32x4_t*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float (&v)[VEC8]) {
    u32x4_t u;
    u.x = f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
    u.y = f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
    u.z = f32_to_bf16_bits(v[4]) | ((uint32_t)f32_to_bf16_bits(v[5]) << 16);
    u.w = f32_to_bf16_bits(v[6]) | ((uint32_t)f32_to_bf16_bits(v[7]) << 16);
    *reinterpret_cast<u32x4_t*>(p) = u;
  }
};
