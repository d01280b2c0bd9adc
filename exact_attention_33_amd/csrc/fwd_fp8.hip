// Fused prefill attention on fp8 (OCP E4M3) q, k, v for gfx950 (D = 64, 128).
//
// FlashAttention-3 takes the attention products to low-precision FP8
// (FlashAttention explainer, aiunderstanding.org, "The future of
// FlashAttention" and the FAQ entry on FlashAttention-3; FlashAttention-3
// article, ybx.com, "FA3 innovations" point 3).  Here q, k and v are e4m3
// codes with one descale factor each; the result is the attention of the
// dequantized values, with o in bf16 and lse in fp32.
//
// Same decomposition as the bf16 kernel (8 wavefronts x 32 query rows, K/V
// tiles of 128 keys in two LDS slots loaded by LDS DMA, one barrier per
// tile), with gfx950's fp8 matrix instruction:
//   * S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales):
//     A = 32 keys x 64 dims of K from LDS (32 bytes per lane), B = 64 dims x
//     32 queries of q held in registers.  Both operands hold, in lane half h,
//     the 32 bytes of dims 64t + 32h ...; the instruction pairs byte j of
//     half h of A with byte j of half h of B.
//   * the probabilities are rounded to e4m3 (v_cvt_pk_fp8_f32, round to
//     nearest even) and O^T += V^T P^T runs on the same instruction over 64
//     keys: B = the lane's own 32 probabilities.  For that, the rows of a K
//     tile are permuted in LDS so that the two 32-key score blocks of a
//     64-key group leave lane half h holding keys 32h .. 32h+31 of the group
//     in order; the V^T operand (32 dims x those 32 keys) is then four
//     transposing byte reads (ds_read_b64_tr_b8) of the row-major V tile.
//   * softmax as in the bf16 kernel (base 2, lazy rescale), with the score
//     scale times both descale factors folded into one constant; o is
//     multiplied by the v descale at the end.
#include "common.h"
#include "kernels.h"

namespace ea {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2v __attribute__((ext_vector_type(2)));

struct Fp8Args {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
  uint16_t* o;
  float* lse;
  int B, Hq, Hkv, Sq, Sk;
  int causal, window;
  float c2;        // scale * q_descale * k_descale * log2(e)
  float v_descale;
  int n_qtiles;
  int xcd_heads;
};

constexpr float kSlackP8 = 256.0f;      // largest probability before a rescale

__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  // formats 0/0 = E4M3 for both operands; block scales 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Eight bytes of a transposing LDS read: in each group of 16 lanes, lane i
// receives byte i%8 of the 8-byte chunks addressed by lanes i/8 + 2k, k = 0..7.
__device__ __forceinline__ i32x2v lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2v*)(const lds_void*)p);
}

// Key held by LDS row R of a K tile.  Within each 64-key group, row 32b + m
// (b = score block, m = MFMA output row) holds key 32*hh + 16*b + r, where the
// MFMA output row m = 8*(r/4) + 4*hh + r%4 is element r of lane half hh; so
// lane half hh ends up with keys 32hh .. 32hh+31 of the group, in order.
__device__ __forceinline__ int k8_row_key(int R) {
  const int grp = R >> 6, b = (R >> 5) & 1, m = R & 31;
  const int hh = (m >> 2) & 1, r = 4 * (m >> 3) + (m & 3);
  return 64 * grp + 32 * hh + 16 * b + r;
}

template <int D, int BN, int NW>
__global__ __launch_bounds__(64 * NW, 2) void fwd_fp8_kernel(Fp8Args a) {
  static_assert(D == 64 || D == 128, "head dims 64 and 128");
  constexpr int BM = 32 * NW;          // query rows per workgroup
  static_assert(BN % 64 == 0, "whole 64-key groups");
  constexpr int NDB = D / 32;          // 32-dim blocks of O
  constexpr int NKT = D / 64;          // k-steps of S (64 dims each)
  constexpr int RS = D + 16;           // padded LDS row (bytes) of K and V tiles
  constexpr int RU = RS / 16;          // 16-byte units per row
  constexpr int SLOT = BN * RS;        // one K or V tile
  constexpr int NB = 2 * SLOT / 1024;  // 1 KB DMA blocks per (K, V) tile pair
  constexpr int NBW = (NB + NW - 1) / NW;
  static_assert(SLOT % 1024 == 0, "whole blocks");
  __shared__ __attribute__((aligned(1024))) char sK[2 * SLOT];
  __shared__ __attribute__((aligned(1024))) char sV[2 * SLOT];

  // ---- which (b, h, query tile) ------------------------------------------
  const int BH = a.B * a.Hq;
  int bh, rank;
  if (a.xcd_heads > 0) {
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    bh = xcd * a.xcd_heads + slot % a.xcd_heads;
    rank = slot / a.xcd_heads;
  } else {
    bh = blockIdx.x % BH;
    rank = blockIdx.x / BH;
  }
  const int qtile = a.causal ? (a.n_qtiles - 1 - rank) : rank;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  const int off = a.Sk - a.Sq;
  const int w = a.window;

  const int r0 = qtile * BM, r1 = min(r0 + BM, a.Sq) - 1;
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
  const uint8_t* kh = a.k + kv_base * D;
  const uint8_t* vh = a.v + kv_base * D;

  const int qw0 = r0 + wave * 32;
  const int qw1 = min(qw0 + 31, a.Sq - 1);
  const int qi = qw0 + l32;
  const bool q_ok = qi < a.Sq;
  const int pos = qi + off;
  const int plo = qw0 + off, phi = qw1 + off;
  int key_lo = 0, key_hi = a.Sk - 1;
  if (a.causal) key_hi = min(key_hi, pos);
  if (w >= 0) {
    key_lo = max(key_lo, pos - w);
    key_hi = min(key_hi, pos + w);
  }

  // ---- q (B operand): for k-step t, half hh holds dims 64t + 32hh .. +31 ---
  i32x8 qf[NKT];
  {
    const uint8_t* qrow = a.q + (q_base + (q_ok ? qi : 0)) * D;
#pragma unroll
    for (int t = 0; t < NKT; ++t) {
      const u32x4 z = {0, 0, 0, 0};
      const u32x4 lo = q_ok ? *(const u32x4*)(qrow + 64 * t + 32 * hh) : z;
      const u32x4 hi = q_ok ? *(const u32x4*)(qrow + 64 * t + 32 * hh + 16) : z;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        qf[t][i] = (int)lo[i];
        qf[t][4 + i] = (int)hi[i];
      }
    }
  }

  // ---- tile loads: block bb < SLOT/1024 is a K block, the rest V blocks ----
  uint32_t doff[NBW], ddst[NBW];
  bool disk[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int bb = i * NW + wave;
    disk[i] = bb < SLOT / 1024;
    const int p = (disk[i] ? bb : bb - SLOT / 1024) * 64 + lane;
    const int row = p / RU, u = p % RU;
    const int key = disk[i] ? k8_row_key(row) : row;
    doff[i] = (u < D / 16 && row < BN) ? (uint32_t)(key * D + u * 16) : 0x7ffffff0u;
    ddst[i] = (uint32_t)((disk[i] ? bb : bb - SLOT / 1024) * 1024);
  }
  const int nbw = (NB - wave + NW - 1) / NW;
  const uint32_t sK0 = lds_addr(sK), sV0 = lds_addr(sV);
  auto issue = [&](int tile) {
    const int kt = tile * BN;
    const uint32_t bytes = (uint32_t)(min(BN, a.Sk - kt) * D);
    const auto rk = make_rsrc(kh + (size_t)kt * D, bytes);
    const auto rv = make_rsrc(vh + (size_t)kt * D, bytes);
    const uint32_t kdst = sK0 + (tile & 1) * SLOT, vdst = sV0 + (tile & 1) * SLOT;
#pragma unroll
    for (int i = 0; i < NBW - 1; ++i) dma16(disk[i] ? rk : rv, doff[i], (disk[i] ? kdst : vdst) + ddst[i]);
    if (NB % NW == 0 || nbw == NBW)
      dma16(disk[NBW - 1] ? rk : rv, doff[NBW - 1], (disk[NBW - 1] ? kdst : vdst) + ddst[NBW - 1]);
  };

  // ---- operand addresses inside a tile -------------------------------------
  // K (A of S^T): lane (m = l32, hh) reads row m of a 32-row block, bytes
  // 64t + 32hh .. +31.
  const uint32_t ka = (uint32_t)(l32 * RS + 32 * hh);
  // V^T (A of O^T) for a 64-key group: read c (keys 8c .. 8c+7 of the lane
  // half) supplies, from lane i of each 16-lane group, the 8-byte chunk of
  // row 32*hh + 8c + (i%16)/2 at dims 16*((lane/16)%2) + 8*(i%2) (+ 32*db).
  const uint32_t vt = (uint32_t)((32 * hh + ((lane & 15) >> 1)) * RS + 16 * ((lane >> 4) & 1) + 8 * (lane & 1));

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = kNegInf, l_run = 0.f;
  const float c2 = a.c2;

  // one 64-key group: S for its two 32-key blocks, softmax, P -> e4m3, PV
  auto group = [&](int slot, int kg0, int grp) {
    const char* kb = sK + slot * SLOT + grp * 64 * RS;
    const char* vb = sV + slot * SLOT + grp * 64 * RS;
    f32x16 st[2];
#pragma unroll
    for (int bk = 0; bk < 2; ++bk) {
      st[bk] = f32x16{};
#pragma unroll
      for (int t = 0; t < NKT; ++t) {
        const char* p = kb + bk * 32 * RS + ka + 64 * t;
        const u32x4 lo = *(const u32x4*)p;
        const u32x4 hi = *(const u32x4*)(p + 16);
        i32x8 kf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          kf[i] = (int)lo[i];
          kf[4 + i] = (int)hi[i];
        }
        st[bk] = mfma_fp8(kf, qf[t], st[bk]);
      }
    }
    // element r of block bk in lane half hh holds key kg0 + 32*hh + 16*bk + r
    const bool full = (kg0 + 63 < a.Sk) && (!a.causal || kg0 + 63 <= plo) &&
                      (w < 0 || ((kg0 >= phi - w) && (kg0 + 63 <= plo + w)));
    if (!full) {
      const int lo = key_lo - kg0 - 32 * hh, hi = key_hi - kg0 - 32 * hh;
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = 16 * bk + r;
          st[bk][r] = ((c >= lo) & (c <= hi)) ? st[bk][r] : kNegInf;
        }
    }
    // Probabilities against the running max as it stands: while no p
    // exceeds 2^8 (the rescale slack) the row max need not be known.  A row
    // that has seen no key yet, or a sum above 2^8, takes the exact path:
    // row max, rescale of O and l when it rose by more than the slack,
    // probabilities again.
    float rs = 0.f;
    i32x8 pf;   // byte j = probability of key kg0 + 32*hh + j, e4m3
    auto probs = [&](float m_use) {
      rs = 0.f;
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; r += 4) {
          const float p0 = fast_exp2(__builtin_fmaf(st[bk][r + 0], c2, -m_use));
          const float p1 = fast_exp2(__builtin_fmaf(st[bk][r + 1], c2, -m_use));
          const float p2 = fast_exp2(__builtin_fmaf(st[bk][r + 2], c2, -m_use));
          const float p3 = fast_exp2(__builtin_fmaf(st[bk][r + 3], c2, -m_use));
          rs += (p0 + p1) + (p2 + p3);
          int word = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, 0, false);
          word = __builtin_amdgcn_cvt_pk_fp8_f32(p2, p3, word, true);
          pf[(16 * bk + r) >> 2] = word;
        }
    };
    probs(m_run);
    if (__any((m_run == kNegInf) | (rs > kSlackP8))) {
      float mx = kNegInf;
#pragma unroll
      for (int bk = 0; bk < 2; ++bk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[bk][r]);
      mx = max_swap32(mx) * c2;
      // move to the exact max (not only past the slack), so that rows of
      // many moderate scores do not come back to this path
      if (__any(mx > m_run)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        m_run = m_new;
      }
      probs((m_run == kNegInf) ? 0.f : m_run);
    }
    l_run += rs;
    // O^T += V^T P^T over the group's 64 keys
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      i32x8 vf;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const i32x2v x = lds_read_tr8(vb + vt + (8 * c) * RS + 32 * db);
        vf[2 * c] = x[0];
        vf[2 * c + 1] = x[1];
      }
      oacc[db] = mfma_fp8(vf, pf, oacc[db]);
    }
  };

  // ---- main loop: tile t+1 flies while tile t is multiplied ---------------
  if (t_begin < t_end) issue(t_begin);
  for (int tile = t_begin; tile < t_end; ++tile) {
    wait_vmcnt<0>();
    __syncthreads();
    if (tile + 1 < t_end) issue(tile + 1);
    const int kt0 = tile * BN;
#pragma unroll
    for (int grp = 0; grp < BN / 64; ++grp) {
      // skip a 64-key group no row of this wavefront can see
      const int k0 = kt0 + 64 * grp, k1 = k0 + 63;
      bool any = k0 < a.Sk;
      if (a.causal) any = any && (k0 <= phi);
      if (w >= 0) any = any && (k0 <= phi + w) && (k1 >= plo - w);
      if (any) group(tile & 1, k0, grp);
    }
  }

  // ---- epilogue: o = v_descale * acc / l in bf16, lse in natural log -------
  const float l_tot = sum_swap32(l_run);
  const float inv = (l_tot > 0.f) ? a.v_descale / l_tot : 0.f;
  uint16_t* orow = a.o + (q_base + (q_ok ? qi : 0)) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_row32_bf16(orow + db * 32, oacc[db], inv, hh, q_ok);
  if (q_ok && a.lse != nullptr && hh == 0)
    a.lse[q_base + qi] = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, uint16_t* o, float* lse,
                          const FwdShape& s, float q_descale, float k_descale, float v_descale,
                          hipStream_t stream) {
  Fp8Args a;
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
  a.c2 = s.scale * q_descale * k_descale * kLog2e;
  a.v_descale = v_descale;
  // 8 wavefronts of 32 rows; 4 for a sliding window at D = 64 (see the bf16 launcher)
  const bool narrow = (s.D == 64) && (s.window >= 0);
  const int bm = narrow ? 128 : 256;
  a.n_qtiles = (s.Sq + bm - 1) / bm;
  const int BH = s.B * s.Hq;
  const int64_t nblocks = (int64_t)a.n_qtiles * BH;
  a.xcd_heads = (BH % 8 == 0) ? BH / 8 : 0;
  // 128-key tiles at both head dims: at D = 64, 64-key tiles would load
  // 384 rather than 512 keys for a +-64 window around 256 rows, but measured
  // slower (twice the barriers and DMA rounds per byte)
  if (s.D == 128)
    hipLaunchKernelGGL((fwd_fp8_kernel<128, 128, 8>), dim3((unsigned)nblocks), dim3(512), 0, stream, a);
  else
    if (narrow)
      hipLaunchKernelGGL((fwd_fp8_kernel<64, 128, 4>), dim3((unsigned)nblocks), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((fwd_fp8_kernel<64, 128, 8>), dim3((unsigned)nblocks), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ea
