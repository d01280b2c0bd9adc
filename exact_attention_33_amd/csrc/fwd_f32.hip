// Fused prefill attention on fp32 tensors: fp32 FMAs on the vector ALUs (no
// matrix cores, nothing rounded to bf16), online softmax in base 2, the same
// causal / sliding-window / GQA semantics as the bf16 kernel.
//
// One workgroup = 2 wavefronts = 64 query rows of one (b, h).  Each query row
// is owned by a lane pair (lane, lane ^ 32): each lane keeps half of the row's
// dimensions of q and of the output accumulator in registers; a dot product
// is the sum of the two halves (one lane swap).  K and V tiles of 32 keys are
// staged in LDS (every lane of a half reads the same address: broadcast).
#include "common.h"
#include "kernels.h"

namespace ea {
namespace {

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, Hq, Hkv, Sq, Sk;
  int causal, window;
  float c2;  // scale * log2(e)
  int n_qtiles;
};

constexpr int kRows = 64;
constexpr int kTile = 32;

template <int D>
__global__ __launch_bounds__(128) void fwd_f32_kernel(F32Args a) {
  constexpr int DH = D / 2;  // dimensions per lane
  __shared__ __attribute__((aligned(16))) float sK[kTile * D];
  __shared__ __attribute__((aligned(16))) float sV[kTile * D];

  const int BH = a.B * a.Hq;
  const int bh = blockIdx.x % BH;
  const int qtile = blockIdx.x / BH;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5;
  const int off = a.Sk - a.Sq;
  const int w = a.window;

  const int r0 = qtile * kRows;
  const int r1 = min(r0 + kRows, a.Sq) - 1;
  int kv_lo = 0, kv_hi = a.Sk;
  if (a.causal) kv_hi = min(kv_hi, r1 + off + 1);
  if (w >= 0) {
    kv_lo = max(kv_lo, r0 + off - w);
    kv_hi = min(kv_hi, r1 + off + w + 1);
  }

  const size_t q_base = ((size_t)b * a.Hq + h) * (size_t)a.Sq;
  const size_t kv_base = ((size_t)b * a.Hkv + g) * (size_t)a.Sk;
  const int qi = r0 + wave * 32 + (lane & 31);
  const bool q_ok = qi < a.Sq;
  const int pos = qi + off;

  float qv[DH], acc[DH];
  {
    const float* qrow = a.q + (q_base + (q_ok ? qi : 0)) * D + hh * DH;
#pragma unroll
    for (int d = 0; d < DH; ++d) {
      qv[d] = q_ok ? qrow[d] : 0.f;
      acc[d] = 0.f;
    }
  }
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.c2;

  for (int kt = (kv_hi > kv_lo ? kv_lo : kv_hi); kt < kv_hi; kt += kTile) {
    // stage keys [kt, kt + kTile) of k and v
    for (int e = tid; e < kTile * D / 4; e += 128) {
      const int row = e / (D / 4), c4 = e % (D / 4);
      const int key = kt + row;
      f32x4 kk = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (key < kv_hi) {
        kk = *(const f32x4*)(a.k + (kv_base + key) * D + 4 * c4);
        vv = *(const f32x4*)(a.v + (kv_base + key) * D + 4 * c4);
      }
      *(f32x4*)(sK + row * D + 4 * c4) = kk;
      *(f32x4*)(sV + row * D + 4 * c4) = vv;
    }
    __syncthreads();

    float s[kTile];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const float* kr = sK + j * D + hh * DH;
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < DH; ++d) part = __builtin_fmaf(qv[d], kr[d], part);
      float dot = part + xor_shfl(part, 32);
      const int key = kt + j;
      bool vis = key < kv_hi;
      if (a.causal) vis = vis && key <= pos;
      if (w >= 0) vis = vis && key >= pos - w && key <= pos + w;
      s[j] = vis ? dot * c2 : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int d = 0; d < DH; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < kTile; ++j) {
      const float p = fast_exp2(s[j] - m_use);
      rs += p;
      const float* vr = sV + j * D + hh * DH;
#pragma unroll
      for (int d = 0; d < DH; ++d) acc[d] = __builtin_fmaf(p, vr[d], acc[d]);
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
    __syncthreads();
  }

  if (q_ok) {
    const float inv = (l_run > 0.f) ? 1.f / l_run : 0.f;
    float* orow = a.o + (q_base + qi) * D + hh * DH;
#pragma unroll
    for (int d = 0; d < DH; d += 4) {
      f32x4 ov = {acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv};
      *(f32x4*)(orow + d) = ov;
    }
    if (a.lse != nullptr && hh == 0)
      a.lse[q_base + qi] = (l_run > 0.f) ? (m_run + __log2f(l_run)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const FwdShape& s, hipStream_t stream) {
  F32Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.Sq = s.Sq;
  a.Sk = s.Sk;
  a.causal = s.causal;
  a.window = s.window;
  a.c2 = s.scale * kLog2e;
  a.n_qtiles = (s.Sq + kRows - 1) / kRows;
  dim3 grid((unsigned)((int64_t)a.n_qtiles * s.B * s.Hq)), block(128);
  if (s.D == 128)
    hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace ea
