// Fused prefill attention on fp32 tensors: fp32 FMAs on the vector ALUs (no
// matrix cores, nothing rounded to bf16), online softmax in base 2, the same
// causal / sliding-window / GQA semantics as the bf16 kernel.
//
// Built for latency (the fp32 workload is a single 128 x 128 head, so the
// work per lane, not the chip's throughput, sets the time): one workgroup =
// NW = 16 wavefronts serving 16 query rows of one (b, h).  Each query row is
// owned by four lanes (row = lane % 16, quarter = lane / 16) in every
// wavefront; each lane keeps a quarter of the row's dimensions of q and of
// its accumulator, and a dot product is the sum of the four quarters (two
// lane exchanges).  K and V blocks of KT keys are staged in LDS by the whole
// workgroup; wavefront w takes keys w, w + NW, ... of each block, so all NW
// wavefronts work on every block at once.  At the end the NW partial results
// (m, l, acc) of each row are merged through LDS with the log-sum-exp
// operator -- the merge of the Tree Attention abstract (express24.ir page),
// here across the wavefronts of one workgroup -- wavefront r merging row r,
// one output dimension (or two) per lane.
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

constexpr int kRows = kF32Rows;       // query rows per workgroup (= lanes per quarter)
constexpr int kNW = kF32Threads / 64;  // wavefronts per workgroup

template <int D>
__global__ __launch_bounds__(64 * kNW) void fwd_f32_kernel(F32Args a) {
  constexpr int DQ = D / 4;                 // dimensions per lane
  constexpr int KT = (D == 64) ? 128 : 64;  // keys per LDS block (64 KB of K and V)
  constexpr int MS = D + 4;                 // floats per (wavefront, row) partial, 16-byte rows
  constexpr int NJ = KT / kNW;              // keys per wavefront and block
  static_assert(KT % kNW == 0, "whole keys per wavefront");
  static_assert(kNW == kRows, "wavefront r merges row r");
  // K/V blocks during the loop, the partials of the merge afterwards
  constexpr int NF = (2 * KT * D > kNW * kRows * MS) ? 2 * KT * D : kNW * kRows * MS;
  __shared__ __attribute__((aligned(16))) float smem[NF];
  float* sK = smem;
  float* sV = smem + KT * D;

  const int BH = a.B * a.Hq;
  const int bh = blockIdx.x % BH;
  const int qtile = blockIdx.x / BH;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = lane & 15, quarter = lane >> 4;
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
  const int qi = r0 + row;
  const bool q_ok = qi < a.Sq;
  const int pos = qi + off;
  int key_lo = 0, key_hi = a.Sk - 1;  // keys this row sees
  if (a.causal) key_hi = min(key_hi, pos);
  if (w >= 0) {
    key_lo = max(key_lo, pos - w);
    key_hi = min(key_hi, pos + w);
  }

  float qv[DQ], acc[DQ];
  {
    const float* qrow = a.q + (q_base + (q_ok ? qi : 0)) * D + quarter * DQ;
#pragma unroll
    for (int d = 0; d < DQ; d += 4) {
      const f32x4 x = q_ok ? *(const f32x4*)(qrow + d) : f32x4{0, 0, 0, 0};
      qv[d] = x[0];
      qv[d + 1] = x[1];
      qv[d + 2] = x[2];
      qv[d + 3] = x[3];
    }
#pragma unroll
    for (int d = 0; d < DQ; ++d) acc[d] = 0.f;
  }
  float m_run = kNegInf, l_run = 0.f;  // base-2 units
  const float c2 = a.c2;

  for (int kt = (kv_hi > kv_lo ? kv_lo : kv_hi); kt < kv_hi; kt += KT) {
    // stage keys [kt, kt + KT) of k and v (zeros past kv_hi)
    for (int e = tid; e < KT * D / 4; e += 64 * kNW) {
      const int key_row = e / (D / 4), c4 = e % (D / 4);
      const int key = kt + key_row;
      f32x4 kk = {0, 0, 0, 0}, vv = {0, 0, 0, 0};
      if (key < kv_hi) {
        kk = *(const f32x4*)(a.k + (kv_base + key) * D + 4 * c4);
        vv = *(const f32x4*)(a.v + (kv_base + key) * D + 4 * c4);
      }
      *(f32x4*)(sK + key_row * D + 4 * c4) = kk;
      *(f32x4*)(sV + key_row * D + 4 * c4) = vv;
    }
    __syncthreads();

    // this wavefront's keys of the block: kt + wave + kNW * j
    float s[NJ];
    float mx = kNegInf;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int key_row = wave + kNW * j;
      const float* kr = sK + key_row * D + quarter * DQ;
      float part = 0.f;
#pragma unroll
      for (int d = 0; d < DQ; ++d) part = __builtin_fmaf(qv[d], kr[d], part);
      part += xor_shfl(part, 16);
      const float dot = sum_swap32(part);
      const int key = kt + key_row;
      const bool vis = (key < kv_hi) & (key >= key_lo) & (key <= key_hi);
      s[j] = vis ? dot * c2 : kNegInf;
      mx = fmaxf(mx, s[j]);
    }
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int d = 0; d < DQ; ++d) acc[d] *= alpha;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const float p = fast_exp2(s[j] - m_use);
      rs += p;
      const float* vr = sV + (wave + kNW * j) * D + quarter * DQ;
#pragma unroll
      for (int d = 0; d < DQ; ++d) acc[d] = __builtin_fmaf(p, vr[d], acc[d]);
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
    __syncthreads();
  }

  // the kNW partials of each row: partial (wave, row) at
  // smem[(wave * kRows + row) * MS], acc[D] then m, l
  {
    float* pm = smem + (wave * kRows + row) * MS;
#pragma unroll
    for (int d = 0; d < DQ; d += 4)
      *(f32x4*)(pm + quarter * DQ + d) = f32x4{acc[d], acc[d + 1], acc[d + 2], acc[d + 3]};
    if (quarter == 0) {
      pm[D] = m_run;
      pm[D + 1] = l_run;
    }
  }
  __syncthreads();

  // wavefront r merges row r: lane l holds output dimensions l (and l + 64)
  {
    const int mrow = wave, mqi = r0 + mrow;
    constexpr int DPL = D / 64;  // output dimensions per lane
    float M = kNegInf;
#pragma unroll
    for (int u = 0; u < kNW; ++u) M = fmaxf(M, smem[(u * kRows + mrow) * MS + D]);
    const float mref = (M == kNegInf) ? 0.f : M;
    float out[DPL], L = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) out[i] = 0.f;
#pragma unroll
    for (int u = 0; u < kNW; ++u) {
      const float* pm = smem + (u * kRows + mrow) * MS;
      const float mu = pm[D];
      const float f = (mu == kNegInf) ? 0.f : fast_exp2(mu - mref);
      L = __builtin_fmaf(pm[D + 1], f, L);
#pragma unroll
      for (int i = 0; i < DPL; ++i) out[i] = __builtin_fmaf(pm[lane + 64 * i], f, out[i]);
    }
    if (mqi < a.Sq) {
      const float inv = (L > 0.f) ? 1.f / L : 0.f;
      float* orow = a.o + (q_base + mqi) * D;
#pragma unroll
      for (int i = 0; i < DPL; ++i) orow[lane + 64 * i] = out[i] * inv;
      if (a.lse != nullptr && lane == 0) a.lse[q_base + mqi] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : kNegInf;
    }
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
  dim3 grid((unsigned)((int64_t)a.n_qtiles * s.B * s.Hq)), block(64 * kNW);
  if (s.D == 128)
    hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace ea
