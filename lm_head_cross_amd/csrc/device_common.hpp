// Shared device types and numerics for the fused linear cross-entropy kernels
// (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define FLCE_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Per-call metadata kept at the start of the workspace.
struct Meta {
  int32_t n_valid;   // number of positions whose label is not ignore_index (Tv)
  int32_t reserved[63];
};

// exp(x) through the hardware base-2 exponential.
__device__ __forceinline__ float exp_e(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

// Natural log through the hardware base-2 logarithm.
__device__ __forceinline__ float log_e(float x) { return __builtin_amdgcn_logf(x) * kLn2; }

// Logit softcap z' = c tanh(z / c) ("nemo_automodel.components.models.
// inkling2.loss", class description: the softcap is fp32 arithmetic).
// tanh(y) = 1 - 2 / (1 + e^{2y}), with e^{2y} from the hardware base-2
// exponential (k2 = 2 log2(e) / c) and one hardware reciprocal: for y > 44,
// e^{2y} = inf and the quotient is 0 (tanh = 1); for y < -44 it is 2
// (tanh = -1).  The absolute error is a few fp32 ulps of 1, about 2e-6 in
// z' for c = 30.  softcap_recip returns 1 / (1 + e^{2y}); the epilogues fold
// the rest (c (1 - 2 r), or 1 - 2 r) into one fma.
__device__ __forceinline__ float softcap_recip(float z, float k2) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * k2));
}

// Merge two (max, sum of exp(x - max)) pairs; a max of -inf means "empty".
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mx = __builtin_fmaxf(m, m2);
  if (mx == kNegInf) return;
  s = s * exp_e(m - mx) + s2 * exp_e(m2 - mx);
  m = mx;
}

__device__ __forceinline__ float lane_xor32(float v) {
  // Swap the two 32-lane halves of the wave.
  return __shfl_xor(v, 32, 64);
}

}  // namespace flce
