// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// 2^x on the transcendental unit (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Value of lane (lane ^ mask) within the wavefront.
__device__ __forceinline__ float xor_shfl(float x, int mask) { return __shfl_xor(x, mask, 64); }

// Two bf16 (low halves / high halves of two packed words) into one word:
// result.lo = x.half, result.hi = y.half.
__device__ __forceinline__ uint32_t pack_lo(uint32_t x, uint32_t y) {
  return (x & 0xffffu) | (y << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t x, uint32_t y) {
  return (x >> 16) | (y & 0xffff0000u);
}

// i-th bf16 (0..7) pair-packed from word i/2 of two 16-byte vectors.
__device__ __forceinline__ uint32_t pick_pair(const u32x4& x, const u32x4& y, int i) {
  return (i & 1) ? pack_hi(x[i >> 1], y[i >> 1]) : pack_lo(x[i >> 1], y[i >> 1]);
}

// Log-sum-exp merge of two partials in base-2 units: (m, l) pairs and the
// factors that scale each side's accumulator.  A side with m = -inf
// contributes nothing.
struct MergeFactors {
  float m, fa, fb;
};
__device__ __forceinline__ MergeFactors merge_factors(float ma, float mb) {
  MergeFactors r;
  r.m = fmaxf(ma, mb);
  const float ref = (r.m == kNegInf) ? 0.f : r.m;
  r.fa = (ma == kNegInf) ? 0.f : fast_exp2(ma - ref);
  r.fb = (mb == kNegInf) ? 0.f : fast_exp2(mb - ref);
  return r;
}

}  // namespace ea
