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
// XCD-aware block remap. The hardware hands consecutive workgroup ids to the
// 8 XCDs round-robin; remapping makes a run of consecutive *logical* tiles
// land on one XCD, so tiles that share weights share that XCD's L2.

__device__ __forceinline__ uint32_t xcd_remap(uint32_t bid, uint32_t nblocks) {
  const uint32_t nx = 8;
  uint32_t per = nblocks / nx;         // full rounds
  uint32_t rem = nblocks % nx;
  uint32_t xcd = bid % nx;
  uint32_t slot = bid / nx;
  // XCDs [0, rem) own per+1 logical blocks, the rest own per.
  uint32_t base = xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per;
  return base + slot;
}
