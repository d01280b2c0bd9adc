// Fused prefill attention for gfx950: bf16 MFMA for q k^T and p v, fp32
// online softmax, causal / sliding-window / GQA.  The score tile lives in
// registers only; nothing of size Sq x Sk ever reaches memory (FlashAttention
// explainer, aiunderstanding.org, "Technical insight": blocks of q, k, v are
// staged in on-chip memory, partial results are rescaled as each new block
// arrives, and the whole computation is one fused kernel).
//
// Work decomposition
//   * one workgroup = 4 wavefronts = BM = 128 query rows of one (b, h);
//     each wavefront owns 32 rows.  K and V tiles of BN keys are staged in
//     LDS once per workgroup and read by all four wavefronts.
//   * scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_32x32x16_bf16: A = 32 keys x 16 dims (from LDS),
//     B = 16 dims x 32 queries (Q fragment held in registers for the whole
//     kernel).  In the accumulator each lane then holds ONE query (its lane
//     mod 32) and 16 of the block's 32 keys, so the row max and row sum are
//     mostly in-lane; one lane-swap (lane ^ 32) finishes the max.
//   * the output is computed transposed too, O^T += V^T P^T: A = 32 dims x
//     16 keys of V^T (LDS), B = the lane's own probabilities converted to
//     bf16 -- no data movement between lanes.  This works because K rows are
//     stored in LDS in a permuted order (bits 2 and 3 of the key index
//     swapped within each 32-key block), which makes the 8 keys a lane holds
//     for each 16-key step of the p v product contiguous.
//   * V is stored in LDS transposed ([d][key]) so that the 8 keys an MFMA
//     operand needs for one d are one 16-byte read; the transpose happens in
//     registers while storing (pairs of bf16 from different keys are packed
//     into one word).
//   * LDS layouts are XOR-swizzled on 16-byte chunks so that both the
//     cooperative stores and the MFMA operand reads are free of bank
//     conflicts.
//   * the next K/V tile is fetched from HBM into registers while the current
//     one is being multiplied (register double buffering).
//   * all softmax arithmetic is base 2: scores are multiplied by
//     scale*log2(e) inside one FMA, exponentials use v_exp_f32.
#include "common.h"
#include "kernels.h"

namespace ea {
namespace {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, Sq, Sk;
  int causal, window;
  float c2;  // scale * log2(e)
  int n_qtiles;
  int xcd_heads;  // > 0: heads per XCD for the XCD-aware block order
};

constexpr int kBM = 128;
constexpr int kThreads = 256;

// Position in LDS of key row `r` of a tile: bits 2 and 3 swapped.
__device__ __forceinline__ int key_slot(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <int D, int BN>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int KCH = D / 8;                    // 16-byte chunks per row
  constexpr int KLOADS = BN * KCH / kThreads;   // 16-byte loads per thread per K tile
  constexpr int KPT = BN * KCH / kThreads;      // keys per thread in the V transpose
  constexpr int VGRP = BN / KPT;                // key groups per V tile
  constexpr int NKB = BN / 32;                  // 32-key blocks per tile
  constexpr int NDB = D / 32;                   // 32-dim blocks of the output
  constexpr int NQK = D / 16;                   // k-steps of q k^T
  static_assert(KPT == 2 || KPT == 4, "V transpose packs 2 or 4 keys per thread");
  static_assert(BN % 32 == 0 && BN / 8 >= 8, "V^T rows need >= 8 chunks for the swizzle");

  __shared__ __attribute__((aligned(16))) uint16_t sK[BN * D];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * BN];

  // ---- which (b, h, query tile) this workgroup computes -----------------
  const int BH = a.B * a.Hq;
  int bh, rank;
  if (a.xcd_heads > 0) {
    // Blocks are dispatched round-robin over the 8 XCDs; give each XCD a
    // contiguous set of heads so a head's K/V stays in one L2.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    bh = xcd * a.xcd_heads + slot % a.xcd_heads;
    rank = slot / a.xcd_heads;
  } else {
    bh = blockIdx.x % BH;
    rank = blockIdx.x / BH;
  }
  // causal: heaviest (last) query tiles first, so short tiles fill the tail
  const int qtile = a.causal ? (a.n_qtiles - 1 - rank) : rank;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int g = h / (a.Hq / a.Hkv);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int off = a.Sk - a.Sq;
  const int w = a.window;

  const int r0 = qtile * kBM;
  const int r1 = min(r0 + kBM, a.Sq) - 1;
  int kv_lo = 0, kv_hi = a.Sk;
  if (a.causal) kv_hi = min(kv_hi, r1 + off + 1);
  if (w >= 0) {
    kv_lo = max(kv_lo, r0 + off - w);
    kv_hi = min(kv_hi, r1 + off + w + 1);
  }
  const int t_begin = kv_lo / BN;
  const int t_end = (kv_hi > kv_lo) ? (kv_hi + BN - 1) / BN : t_begin;

  const size_t q_base = ((size_t)b * a.Hq + h) * (size_t)a.Sq;
  const size_t kv_base = ((size_t)b * a.Hkv + g) * (size_t)a.Sk;

  const int qw0 = r0 + wave * 32;               // first row of this wavefront
  const int qw1 = min(qw0 + 31, a.Sq - 1);      // last valid row
  const int qi = qw0 + l32;                     // this lane's row
  const bool q_ok = qi < a.Sq;
  const bool wave_live = qw0 < a.Sq;

  // ---- Q fragment (B operand of S^T = K Q^T) ----------------------------
  bf16x8 qf[NQK];
  {
    const uint16_t* qrow = a.q + (q_base + (q_ok ? qi : 0)) * D;
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
      u32x4 raw = q_ok ? *(const u32x4*)(qrow + 16 * t + 8 * hh) : u32x4{0, 0, 0, 0};
      qf[t] = __builtin_bit_cast(bf16x8, raw);
    }
  }

  // ---- K/V tile fetch (HBM -> registers) and store (registers -> LDS) ----
  u32x4 kr[KLOADS];
  u32x4 vr[KPT];
  const int vkg = tid % VGRP, vch = tid / VGRP;  // V: key group, 16-byte chunk

  auto fetch = [&](int tile) {
    const int kt = tile * BN;
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int e = tid + i * kThreads;
      const int row = e / KCH, ch = e % KCH;
      const int key = kt + row;
      kr[i] = (key < a.Sk) ? *(const u32x4*)(a.k + (kv_base + key) * D + ch * 8) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      const int key = kt + vkg * KPT + e;
      vr[e] = (key < a.Sk) ? *(const u32x4*)(a.v + (kv_base + key) * D + vch * 8) : u32x4{0, 0, 0, 0};
    }
  };

  auto store = [&]() {
#pragma unroll
    for (int i = 0; i < KLOADS; ++i) {
      const int e = tid + i * kThreads;
      const int row = e / KCH, ch = e % KCH;
      const int lrow = key_slot(row);
      const int pch = ch ^ (lrow & 7);
      *(u32x4*)(sK + lrow * D + pch * 8) = kr[i];
    }
    // V^T: row d = 8*vch + i holds this thread's KPT keys at column vkg*KPT
    const int kc = (vkg * KPT) / 8, kin = (vkg * KPT) % 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = vch * 8 + i;
      uint16_t* dst = sV + d * BN + ((kc ^ (d & 7)) * 8) + kin;
      if constexpr (KPT == 4) {
        u32x2 pr;
        pr[0] = pick_pair(vr[0], vr[1], i);
        pr[1] = pick_pair(vr[2], vr[3], i);
        *(u32x2*)dst = pr;
      } else {
        *(uint32_t*)dst = pick_pair(vr[0], vr[1], i);
      }
    }
  };

  // ---- main loop ----------------------------------------------------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = kNegInf;  // running max of c2 * score (base-2 units)
  float l_run = 0.f;      // this lane's part of the running sum (its 16 keys per block)
  const float c2 = a.c2;
  const int pos = qi + off;  // key position aligned with this lane's row

  if (t_begin < t_end) fetch(t_begin);
  for (int tile = t_begin; tile < t_end; ++tile) {
    store();
    __syncthreads();
    if (tile + 1 < t_end) fetch(tile + 1);

    const int kt0 = tile * BN, kt1 = kt0 + BN - 1;
    const int plo = qw0 + off, phi = qw1 + off;
    bool any = wave_live, full = kt1 < a.Sk;
    if (a.causal) {
      any = any && (kt0 <= phi);
      full = full && (kt1 <= plo);
    }
    if (w >= 0) {
      any = any && (kt1 >= plo - w) && (kt0 <= phi + w);
      full = full && (kt0 >= phi - w) && (kt1 <= plo + w);
    }

    if (any) {
      // S^T = K Q^T
      f32x16 st[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        st[kb] = f32x16{};
        const int lrow = kb * 32 + l32;
#pragma unroll
        for (int t = 0; t < NQK; ++t) {
          const int pch = (2 * t + hh) ^ (lrow & 7);
          const bf16x8 kf = *(const bf16x8*)(sK + lrow * D + pch * 8);
          st[kb] = mfma32(kf, qf[t], st[kb]);
        }
      }
      // key of accumulator r in block kb: kt0 + 32kb + 16(r/8) + 8hh + r%8
      if (!full) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kt0 + kb * 32 + 16 * (r >> 3) + 8 * hh + (r & 7);
            bool vis = key < a.Sk;
            if (a.causal) vis = vis && key <= pos;
            if (w >= 0) vis = vis && key >= pos - w && key <= pos + w;
            st[kb][r] = vis ? st[kb][r] : kNegInf;
          }
        }
      }
      // online softmax (base 2)
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
      mx = fmaxf(mx, xor_shfl(mx, 32));
      const float m_new = fmaxf(m_run, mx * c2);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(st[kb][r], c2, -m_use));
          st[kb][r] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;

      // O^T += V^T P^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          bf16x8 pf;
#pragma unroll
          for (int j = 0; j < 8; ++j) pf[j] = (__bf16)st[kb][8 * s + j];
          const int ch = 4 * kb + 2 * s + hh;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const int d = db * 32 + l32;
            const bf16x8 vf = *(const bf16x8*)(sV + d * BN + ((ch ^ (d & 7)) * 8));
            oacc[db] = mfma32(vf, pf, oacc[db]);
          }
        }
      }
    }
    __syncthreads();
  }

  // ---- epilogue: normalise, round once to bf16, write o and lse ----------
  const float l_tot = l_run + xor_shfl(l_run, 32);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  if (q_ok) {
    uint16_t* orow = a.o + (q_base + qi) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 ov;
#pragma unroll
        for (int j = 0; j < 4; ++j) ov[j] = (__bf16)(oacc[db][4 * g4 + j] * inv);
        *(bf16x4*)(orow + db * 32 + 8 * g4 + 4 * hh) = ov;
      }
    }
    if (a.lse != nullptr && hh == 0)
      a.lse[q_base + qi] = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, const FwdShape& s, hipStream_t stream) {
  FwdArgs a;
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
  a.n_qtiles = (s.Sq + kBM - 1) / kBM;
  const int BH = s.B * s.Hq;
  const int64_t nblocks = (int64_t)a.n_qtiles * BH;
  a.xcd_heads = (BH % 8 == 0) ? BH / 8 : 0;
  dim3 grid((unsigned)nblocks), block(kThreads);
  if (s.D == 128)
    hipLaunchKernelGGL((fwd_bf16_kernel<128, 64>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<64, 128>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace ea
