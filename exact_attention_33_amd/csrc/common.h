// Device-side helpers shared by the gfx950 attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) void lds_void;

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

// LDS byte address of a __shared__ object (what M0 and ds_* addresses use).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const lds_void*)p;
}

// Buffer resource over [base, base + bytes): loads past the end return 0.
// Callers pass wave-uniform values; readfirstlane makes that explicit so the
// descriptor always lives in scalar registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = (uint64_t)(uintptr_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  void* pu = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           0x00020000);
}

// One 16-byte-per-lane load from a buffer straight into LDS: lane i's 16
// bytes land at LDS byte address lds_base + 16*i (lds_base wave-uniform).
// Issued from asm so the compiler does not guard later LDS reads with a
// blanket vmcnt(0); completion is awaited explicitly (vmcnt) by the caller.
// The LDS base goes in as an M0 operand ("{m0}"), so the compiler sets M0
// itself before the block and knows its value.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t lds_base) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :: "v"(voff), "s"(rs), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base)) : "memory");
}

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Four bf16 of a transposing LDS read (16-lane groups): lane i of a group
// receives element i%4 of the 8-byte rows addressed by lanes i/4 + 4k, k=0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(const lds_void*)p);
}

// Value of lane (lane ^ mask) within the wavefront.
__device__ __forceinline__ float xor_shfl(float x, int mask) { return __shfl_xor(x, mask, 64); }

// max / sum of x over lanes l and l^32 (v_permlane32_swap, no LDS traffic)
__device__ __forceinline__ float max_swap32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_swap32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Write one 32-column block of a row held in the layout of a 32x32 MFMA
// result whose columns are the rows of the output: lane l has element
// 4g + j (g, j = 0..3) of column 8g + 4*(l/32) + j.  The values are scaled,
// rounded to bf16 and, after one exchange between lanes l and l+32 per pair
// of 4-column chunks (v_permlane32_swap moves lanes 32..63 of its first
// operand and lanes 0..31 of its second), each lane writes 8 consecutive
// columns with one 16-byte store: half the store instructions of 8-byte
// stores, and 32 contiguous bytes per row per instruction.  Every lane must
// call this (the exchange is cross-lane); `ok` gates only the store.
__device__ __forceinline__ void store_row32_bf16(uint16_t* dst, const f32x16& acc, float mul, int hh, bool ok) {
  uint32_t pk[4][2];
#pragma unroll
  for (int g4 = 0; g4 < 4; ++g4) {
    bf16x4 v;
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = (__bf16)(acc[4 * g4 + j] * mul);
    const u32x2 u = __builtin_bit_cast(u32x2, v);
    pk[g4][0] = u[0];
    pk[g4][1] = u[1];
  }
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    // lower lanes keep chunk 2p and receive the partner's chunk 2p; upper
    // lanes keep chunk 2p+1 and receive the partner's chunk 2p+1
    uint32_t x[2], y[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const auto r = __builtin_amdgcn_permlane32_swap(pk[2 * p][w], pk[2 * p + 1][w], false, false);
      x[w] = r[0];
      y[w] = r[1];
    }
    if (ok) {
      const u32x4 v4 = {x[0], x[1], y[0], y[1]};
      *(u32x4*)(dst + 8 * (2 * p + hh)) = v4;
    }
  }
}

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
