// Split-KV decode for gfx950: one query token per (b, head) against a bf16 KV
// cache, the sequence split into chunks whose partials (m, l, acc) are merged
// with the log-sum-exp operator along a balanced binary tree over the chunk
// index -- the sequence-axis tree reduction of the Tree Attention abstract
// (express24.ir page), here on one device.
//
// Split kernel: one workgroup per (chunk, kv head, batch[, group of 16 query
// heads]); when those groups divide evenly over the 8 XCDs, each XCD takes
// whole groups, chunk after chunk.  It streams its chunk of K and V from HBM exactly once and serves
// every query head that shares the kv head (GQA), which keeps the kernel at
// one read of the cache -- the quantity that bounds decode.  Each of the 4
// wavefronts takes every 4th 32-key step of the chunk:
//   * K and V are read with buffer loads over exactly the step's keys inside
//     the chunk: keys past the chunk end read as zero with no branch, and the
//     per-lane offsets are immediates of the load instructions;
//   * s^T = K q^T on v_mfma_f32_16x16x32_bf16, K loaded straight from HBM
//     into the A-operand layout (16 keys x 32 dims, 16 bytes per lane), the
//     query heads as the 16 columns of B (unused columns are zero);
//   * online softmax per head column in base 2 (v_exp_f32);
//   * o^T += V^T p^T on the same instruction: each lane fetches 8 keys x
//     (D/16) dims of V and transposes them in registers into the A operand
//     (8 consecutive keys for one dim), so V needs no LDS round trip; the
//     probabilities are already in the B-operand layout because K rows were
//     loaded in a matching key order.
// The 4 wavefront partials are merged in LDS ((w0+w1)+(w2+w3)) and one
// partial per head is written: acc unnormalised, m in base-2 units.
//
// Combine kernel: one workgroup per (b, h, group of <= 256 partials).  The
// partials are merged level by level: at stride s the partial at index i (i a
// multiple of 2s) absorbs index i+s; an index with no partner passes up
// unchanged.  Strides 1..32 run in registers within a wavefront (64 partials
// each), strides 64 and 128 across the four wavefronts in LDS.  The root is
// normalised (o = acc / l, lse = ln2 * (m + log2 l)) and written, or, above
// 256 partials, written as one partial of the next tree level.
#include "common.h"
#include "kernels.h"

namespace ea {
namespace {

struct SplitArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* po;   // [B*Hq][ns][D] unnormalised accumulators
  float* pml;  // [B*Hq][ns][2] (m in base-2 units, l)
  int B, Hq, Hkv, Sk, ns, L, nhg;
  int xcd_groups;  // B*Hkv*nhg % 8 == 0: XCD-aware block order
  float c2;  // scale * log2(e)
};

template <int D>
__global__ __launch_bounds__(256) void decode_split_kernel(SplitArgs a) {
  constexpr int NT = D / 32;  // k-steps of s^T = K q^T
  constexpr int VE = D / 16;  // dims of V per lane per key; also MFMAs per step of o^T
  __shared__ float sO[4][16][D + 1];  // +1: the per-lane strided stores hit distinct banks
  __shared__ float sM[4][16];
  __shared__ float sL[4][16];

  // (b, kv head, head group) = group.  Blocks are dispatched round-robin over
  // the 8 XCDs; when the groups divide evenly, each XCD streams whole groups,
  // chunk after chunk, so a group's KV goes through one XCD's L2.
  int c, grp;
  if (a.xcd_groups) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    c = slot % a.ns;
    grp = (slot / a.ns) * 8 + xcd;
  } else {
    c = blockIdx.x % a.ns;
    grp = blockIdx.x / a.ns;
  }
  const int g = grp % a.Hkv;
  grp /= a.Hkv;
  const int hg = grp % a.nhg;
  const int b = grp / a.nhg;
  const int G = a.Hq / a.Hkv;
  const int h0 = g * G + hg * 16;
  const int nh = min(16, G - hg * 16);
  const int64_t c0l = (int64_t)c * a.L;
  const int c0 = (int)(c0l < a.Sk ? c0l : a.Sk);
  const int c1 = (int)((c0l + a.L) < a.Sk ? (c0l + a.L) : a.Sk);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hc = lane & 15, q4 = lane >> 4;
  const bool h_ok = hc < nh;

  bf16x8 qf[NT];
  {
    const uint16_t* qrow = a.q + ((size_t)b * a.Hq + h0 + (h_ok ? hc : 0)) * D;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x4 raw = h_ok ? *(const u32x4*)(qrow + 32 * t + 8 * q4) : u32x4{0, 0, 0, 0};
      qf[t] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  const size_t kvb = ((size_t)b * a.Hkv + g) * (size_t)a.Sk;
  f32x4 oacc[VE];
#pragma unroll
  for (int j = 0; j < VE; ++j) oacc[j] = f32x4{};
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.c2;
  // A-operand row i of key block a2 reads key 8*(i/4) + 4*a2 + i%4 of the step,
  // so lane group q4 ends up holding keys 8*q4 .. 8*q4+7 of the step.
  const int krow = 8 * (hc >> 2) + (hc & 3);
  // per-lane byte offsets inside one 32-key step; the rest are immediates
  const uint32_t koff = (uint32_t)((krow * D + 8 * q4) * 2);
  const uint32_t voff = (uint32_t)((8 * q4 * D + VE * hc) * 2);

  // One 32-key step's K and V for this lane.  The buffer covers only the
  // keys of the step that lie inside the chunk, so keys past the chunk end
  // (or a step entirely past it) read as zero without a branch.
  struct StepRegs {
    u32x4 k[2][NT];
    uint32_t v[8][VE / 2];
  };
  auto load_step = [&](StepRegs& r, int kw) {
    const int nk = max(0, min(32, c1 - kw));
    const auto rk = make_rsrc(a.k + (kvb + (size_t)min(kw, c1)) * D, (uint32_t)(nk * D * 2));
    const auto rv = make_rsrc(a.v + (kvb + (size_t)min(kw, c1)) * D, (uint32_t)(nk * D * 2));
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        r.k[a2][t] = __builtin_amdgcn_raw_buffer_load_b128(rk, koff + (4 * a2 * D + 32 * t) * 2, 0, 0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (VE == 8) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rv, voff + e * D * 2, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) r.v[e][i] = x[i];
      } else {
        const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rv, voff + e * D * 2, 0, 0);
#pragma unroll
        for (int i = 0; i < 2; ++i) r.v[e][i] = x[i];
      }
    }
  };

  // scores, online softmax and o^T += V^T p^T for one step (keys >= c1 masked)
  auto compute_step = [&](const StepRegs& r, int kw) {
    // s^T: lane holds head hc and keys kw + 8*q4 + 4*a2 + r
    f32x4 st[2];
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2) {
      st[a2] = f32x4{};
#pragma unroll
      for (int t = 0; t < NT; ++t)
        st[a2] = mfma16(__builtin_bit_cast(bf16x8, r.k[a2][t]), qf[t], st[a2]);
    }
    float mx = kNegInf;
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = kw + 8 * q4 + 4 * a2 + i;
        st[a2][i] = (key < c1) ? st[a2][i] : kNegInf;
        mx = fmaxf(mx, st[a2][i]);
      }
    mx = fmaxf(mx, xor_shfl(mx, 16));
    mx = fmaxf(mx, xor_shfl(mx, 32));
    const float m_new = fmaxf(m_run, mx * c2);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    bf16x8 pf;
    float rs = 0.f;
#pragma unroll
    for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(__builtin_fmaf(st[a2][i], c2, -m_use));
        rs += p;
        pf[4 * a2 + i] = (__bf16)p;
      }
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < VE; ++j) {
      // V^T operand: 8 keys of dim VE*hc + j, key e in element e
      u32x4 t;
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        t[e2] = (j & 1) ? pack_hi(r.v[2 * e2][j >> 1], r.v[2 * e2 + 1][j >> 1])
                        : pack_lo(r.v[2 * e2][j >> 1], r.v[2 * e2 + 1][j >> 1]);
      oacc[j] = mfma16(__builtin_bit_cast(bf16x8, t), pf, oacc[j] * alpha);
    }
  };

  for (int kw = c0 + 32 * wave; kw < c1; kw += 128) {
    StepRegs r;
    load_step(r, kw);
    compute_step(r, kw);
  }

  // lane (hc, q4) holds dims VE*(4*q4 + r) + j of head hc; l summed over q4
  float l_tot = l_run + xor_shfl(l_run, 16);
  l_tot += xor_shfl(l_tot, 32);
  if (q4 == 0) {
    sM[wave][hc] = m_run;
    sL[wave][hc] = l_tot;
  }
#pragma unroll
  for (int j = 0; j < VE; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) sO[wave][hc][VE * (4 * q4 + r) + j] = oacc[j][r];
  __syncthreads();

  for (int it = tid; it < nh * D; it += 256) {
    const int hcx = it / D, d = it % D;
    const MergeFactors f01 = merge_factors(sM[0][hcx], sM[1][hcx]);
    const MergeFactors f23 = merge_factors(sM[2][hcx], sM[3][hcx]);
    const MergeFactors fr = merge_factors(f01.m, f23.m);
    const float o01 = sO[0][hcx][d] * f01.fa + sO[1][hcx][d] * f01.fb;
    const float o23 = sO[2][hcx][d] * f23.fa + sO[3][hcx][d] * f23.fb;
    const size_t slot = ((size_t)b * a.Hq + h0 + hcx) * a.ns + c;
    a.po[slot * D + d] = o01 * fr.fa + o23 * fr.fb;
    if (d == 0) {
      const float l01 = sL[0][hcx] * f01.fa + sL[1][hcx] * f01.fb;
      const float l23 = sL[2][hcx] * f23.fa + sL[3][hcx] * f23.fb;
      a.pml[slot * 2] = fr.m;
      a.pml[slot * 2 + 1] = l01 * fr.fa + l23 * fr.fb;
    }
  }
}

constexpr int kLeaves = 64;   // partials merged in registers by one wavefront
constexpr int kGroup = 256;   // partials merged by one combine workgroup (4 wavefronts)

struct CombineArgs {
  const float* in_o;   // [BH][n][D]
  const float* in_ml;  // [BH][n][2]
  float* out_o;        // next level [BH][ngroups][D] (non-final pass)
  float* out_ml;
  uint16_t* o;         // final: bf16 [BH][D]
  float* lse;          // final: fp32 [BH] or null
  int n, ngroups, final_pass;
};

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}

// One workgroup per (b*h, group of <= 256 partials).  Wavefront w owns leaves
// 64w .. 64w+63 of the group: lane i holds (m, l) of leaf i and, for every
// leaf, this lane's D/64 dims of the accumulator.  The leaves are merged in
// registers level by level (stride 1, 2, ..., 32: leaf i absorbs leaf i+s
// when i is a multiple of 2s); leaves past the end are the merge identity, so
// an unpaired partial passes up unchanged.  The four wavefront roots are then
// merged in LDS at strides 64 and 128, which completes the balanced binary
// tree over the group's partials.
template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int DPL = D / 64;  // dims per lane
  __shared__ float sO[4][D];
  __shared__ float sM[4], sL[4];

  const int grp = blockIdx.x % a.ngroups;
  const int bh = blockIdx.x / a.ngroups;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int base = grp * kGroup + wave * kLeaves;
  const int nl = max(0, min(kLeaves, a.n - base));
  const size_t row0 = (size_t)bh * a.n + base;

  float m = kNegInf, l = 0.f;
  float o[kLeaves][DPL];
#pragma unroll
  for (int i = 0; i < kLeaves; ++i)
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[i][j] = 0.f;
  if (nl > 0) {
    if (lane < nl) {
      m = a.in_ml[(row0 + lane) * 2];
      l = a.in_ml[(row0 + lane) * 2 + 1];
    }
#pragma unroll
    for (int i = 0; i < kLeaves; ++i) {
      const float* src = a.in_o + (row0 + min(i, nl - 1)) * D + lane * DPL;
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[i][j] = (i < nl) ? src[j] : 0.f;
    }
  }

#pragma unroll
  for (int s = 1; s < kLeaves; s *= 2) {
    const float mj = __shfl_down(m, s, 64);
    const float lj = __shfl_down(l, s, 64);
    const MergeFactors f = merge_factors(m, mj);
    const bool leader = (lane & (2 * s - 1)) == 0;
#pragma unroll
    for (int i = 0; i < kLeaves; i += 2 * s) {
      const float fa = lane_value(f.fa, i), fb = lane_value(f.fb, i);
#pragma unroll
      for (int j = 0; j < DPL; ++j) o[i][j] = o[i][j] * fa + o[i + s][j] * fb;
    }
    l = leader ? l * f.fa + lj * f.fb : l;
    m = leader ? f.m : m;
  }

  if (lane == 0) {
    sM[wave] = m;
    sL[wave] = l;
  }
#pragma unroll
  for (int j = 0; j < DPL; ++j) sO[wave][lane * DPL + j] = o[0][j];
  __syncthreads();
  if (wave != 0) return;

  const MergeFactors f01 = merge_factors(sM[0], sM[1]);
  const MergeFactors f23 = merge_factors(sM[2], sM[3]);
  const MergeFactors fr = merge_factors(f01.m, f23.m);
  const float M = fr.m;
  const float L = (sL[0] * f01.fa + sL[1] * f01.fb) * fr.fa + (sL[2] * f23.fa + sL[3] * f23.fb) * fr.fb;
#pragma unroll
  for (int j = 0; j < DPL; ++j) {
    const int d = lane * DPL + j;
    const float acc = (sO[0][d] * f01.fa + sO[1][d] * f01.fb) * fr.fa +
                      (sO[2][d] * f23.fa + sO[3][d] * f23.fb) * fr.fb;
    if (a.final_pass) {
      const __bf16 ob = (__bf16)((L > 0.f) ? acc / L : 0.f);
      a.o[(size_t)bh * D + d] = __builtin_bit_cast(uint16_t, ob);
    } else {
      a.out_o[((size_t)bh * a.ngroups + grp) * D + d] = acc;
    }
  }
  if (lane == 0) {
    if (a.final_pass) {
      if (a.lse != nullptr) a.lse[bh] = (L > 0.f) ? (M + __log2f(L)) * kLn2 : kNegInf;
    } else {
      const size_t slot = (size_t)bh * a.ngroups + grp;
      a.out_ml[slot * 2] = M;
      a.out_ml[slot * 2 + 1] = L;
    }
  }
}

}  // namespace

int64_t decode_partial_slots(int num_splits) {
  int64_t total = num_splits;
  int64_t n = num_splits;
  while (n > kGroup) {
    n = (n + kGroup - 1) / kGroup;
    total += n;
  }
  return total;
}

hipError_t launch_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                         float* lse, const DecodeShape& s, float* ws, hipStream_t stream) {
  const int BH = s.B * s.Hq;
  const int G = s.Hq / s.Hkv;
  SplitArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.po = ws;
  a.pml = ws + (size_t)BH * s.num_splits * s.D;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.Sk = s.Sk;
  a.ns = s.num_splits;
  a.L = (int)(((int64_t)s.Sk + s.num_splits - 1) / s.num_splits);
  a.nhg = (G + 15) / 16;
  a.xcd_groups = ((int64_t)s.B * s.Hkv * a.nhg) % 8 == 0;
  a.c2 = s.scale * kLog2e;
  dim3 grid((unsigned)((int64_t)s.num_splits * s.Hkv * s.B * a.nhg)), block(256);
  if (s.D == 128)
    hipLaunchKernelGGL((decode_split_kernel<128>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((decode_split_kernel<64>), grid, block, 0, stream, a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  const float* in_o = a.po;
  const float* in_ml = a.pml;
  float* next = a.pml + (size_t)BH * s.num_splits * 2;
  int n = s.num_splits;
  for (;;) {
    CombineArgs c;
    c.in_o = in_o;
    c.in_ml = in_ml;
    c.n = n;
    c.ngroups = (n + kGroup - 1) / kGroup;
    c.final_pass = c.ngroups == 1;
    c.out_o = next;
    c.out_ml = next + (size_t)BH * c.ngroups * s.D;
    c.o = o;
    c.lse = lse;
    dim3 cgrid((unsigned)((int64_t)BH * c.ngroups));
    if (s.D == 128)
      hipLaunchKernelGGL((combine_kernel<128>), cgrid, dim3(256), 0, stream, c);
    else
      hipLaunchKernelGGL((combine_kernel<64>), cgrid, dim3(256), 0, stream, c);
    err = hipGetLastError();
    if (err != hipSuccess || c.final_pass) return err;
    in_o = c.out_o;
    in_ml = c.out_ml;
    next = c.out_ml + (size_t)BH * c.ngroups * 2;
    n = c.ngroups;
  }
}

}  // namespace ea
