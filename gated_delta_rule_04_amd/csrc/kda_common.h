// Shared device helpers of the KDA HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Element loads/stores with conversion to/from float32 compute.
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }  // RNE (v_cvt_pk_bf16_f32)

// Two floats as one packed bf16 pair, rounded to nearest even: one
// v_cvt_pk_bf16_f32.  Wider vectors are converted pair by pair: a conversion
// of four lanes at once is otherwise split into four half-empty conversions
// and two permutes.
__device__ __forceinline__ unsigned pk_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4& v) {
  typedef unsigned u32x2p __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(bf16x4, u32x2p{pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3])});
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNormEps = 1e-6f;  // guard of the prologue's L2 normalisation

// Prologue activations (fp32).  The gate's softplus is taken in log2 units:
// with xs = x log2(e), softplus(x) log2(e) = log2(1 + 2^xs), because the ln 2
// of the natural log and the log2(e) of the change of base cancel.  That is
// xs itself above 15 log2(e) and 2^xs log2(e) below -15 log2(e) (where the
// rounded forms are exact to fp32), else the hardware exp2 and log2.  Both
// transcendentals are issued unconditionally and the branch is a select.
__device__ __forceinline__ float softplus_log2(float xs) {
  const float e = fast_exp2(xs);
  const float l = __builtin_amdgcn_logf(1.f + e);
  return xs > 15.f * kLog2e ? xs : (xs < -15.f * kLog2e ? e * kLog2e : l);
}
__device__ __forceinline__ float sigmoid_f(float x) { return 1.f / (1.f + fast_exp2(-x * kLog2e)); }

}  // namespace kda
