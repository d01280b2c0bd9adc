// Reference kernels for measurement (declared in include/attn_calib.h): a
// plain HBM stream and a plain MFMA loop.  They give the achievable rates of
// the part the attention kernels are compared with; nothing here is used by
// the attention path.
#include <stdint.h>

#include "../../include/attn_calib.h"
#include "common.h"

namespace ea {
namespace {

constexpr int kCalibThreads = 256;

// dst chunk j = XOR over r of src chunk j + r*n (n = number of dst chunks).
// Each wavefront owns 256 consecutive dst chunks per pass (four 1 KB rows of
// 64 lanes) and, for each r, loads the four source rows together, so every
// stream is read as one contiguous front moving through memory and each
// thread keeps four or more loads in flight whatever the ratio.
__global__ __launch_bounds__(kCalibThreads) void stream_kernel(const u32x4* __restrict__ src,
                                                               u32x4* __restrict__ dst,
                                                               int64_t n, int64_t reps) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (kCalibThreads / 64) + (threadIdx.x >> 6);
  const int64_t step = (int64_t)gridDim.x * (kCalibThreads / 64) * 256;
  for (int64_t j0 = wave * 256 + lane; j0 < n; j0 += step) {
    u32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = u32x4{0, 0, 0, 0};
#pragma unroll 2
    for (int64_t r = 0; r < reps; ++r) {
      const u32x4* s = src + r * n;
      u32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = (j0 + 64 * u < n) ? s[j0 + 64 * u] : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] ^= x[u];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (j0 + 64 * u < n) dst[j0 + 64 * u] = acc[u];
  }
}

// Four independent accumulation chains per wavefront; operands differ per
// lane and per chain so nothing folds at compile time.
__global__ __launch_bounds__(kCalibThreads) void mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)(lane + i));
    b[i] = (__bf16)(0.002f * (float)(63 - lane + i));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(b, a, c1);
    c2 = mfma32(a, a, c2);
    c3 = mfma32(b, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

typedef int i32x8 __attribute__((ext_vector_type(8)));

// One fp8 matrix instruction on caller-given operands, C = 0, unit block
// scales (E4M3 x E4M3).  Lane l holds row / column l % 32 and the 32 k-values
// 32 * (l / 32) .. + 31 of its A row and B column; result element i of lane l
// is c[8 * (i / 4) + 4 * (l / 32) + i % 4][l % 32].
__global__ __launch_bounds__(64) void mfma_fp8_probe_kernel(const uint8_t* __restrict__ a,
                                                            const uint8_t* __restrict__ b,
                                                            float* __restrict__ c) {
  const int lane = threadIdx.x & 63;
  const int rc = lane & 31, half = lane >> 5;
  const i32x8 av = *(const i32x8*)(a + rc * 64 + 32 * half);
  const i32x8 bv = *(const i32x8*)(b + rc * 64 + 32 * half);
  f32x16 acc = {};
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
#pragma unroll
  for (int i = 0; i < 16; ++i) c[(8 * (i >> 2) + 4 * half + (i & 3)) * 32 + rc] = acc[i];
}

}  // namespace
}  // namespace ea

extern "C" int attn_calib_mfma_fp8(const void* a, const void* b, float* c, hipStream_t stream) {
  if (a == nullptr || b == nullptr || c == nullptr) return ATTN_ERR_NULL;
  if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) % 16 != 0) return ATTN_ERR_ARG;
  hipLaunchKernelGGL(ea::mfma_fp8_probe_kernel, dim3(1), dim3(64), 0, stream, (const uint8_t*)a,
                     (const uint8_t*)b, c);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_calib_stream(const void* src, size_t src_bytes, void* dst, size_t dst_bytes,
                                 hipStream_t stream) {
  if (src_bytes == 0 && dst_bytes == 0) return ATTN_OK;
  if (dst_bytes == 0) return ATTN_ERR_ARG;
  if (dst == nullptr || (src_bytes > 0 && src == nullptr)) return ATTN_ERR_NULL;
  if (src_bytes % 16 != 0 || dst_bytes % 16 != 0 || src_bytes % dst_bytes != 0) return ATTN_ERR_ARG;
  if (((uintptr_t)src | (uintptr_t)dst) % 16 != 0) return ATTN_ERR_ARG;
  const int64_t n = (int64_t)(dst_bytes / 16);
  const int64_t reps = (int64_t)(src_bytes / dst_bytes);
  const int64_t want = (n + 4 * ea::kCalibThreads - 1) / (4 * ea::kCalibThreads);
  const unsigned grid = (unsigned)(want < 16384 ? want : 16384);
  hipLaunchKernelGGL(ea::stream_kernel, dim3(grid), dim3(ea::kCalibThreads), 0, stream,
                     (const ea::u32x4*)src, (ea::u32x4*)dst, n, reps);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" int attn_calib_mfma(float* out, int workgroups, int iters, hipStream_t stream) {
  if (workgroups < 0 || iters < 0 || workgroups > (1 << 20)) return ATTN_ERR_ARG;
  if (workgroups == 0) return ATTN_OK;
  if (out == nullptr) return ATTN_ERR_NULL;
  hipLaunchKernelGGL(ea::mfma_kernel, dim3((unsigned)workgroups), dim3(ea::kCalibThreads), 0, stream, out,
                     iters);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" double attn_calib_mfma_flops(int workgroups, int iters) {
  return 2.0 * 32 * 32 * 16 * 4 * 4 * (double)iters * (double)workgroups;
}
