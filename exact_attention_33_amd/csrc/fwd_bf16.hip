// Fused prefill attention for gfx950: bf16 MFMA for q k^T and p v, fp32
// online softmax, causal / sliding-window / GQA.  The score tile lives in
// registers only; nothing of size Sq x Sk ever reaches memory (FlashAttention
// explainer, aiunderstanding.org, "Technical insight": blocks of q, k, v are
// staged in on-chip memory, partial results are rescaled as each new block
// arrives, and the whole computation is one fused kernel).  Data movement is
// overlapped with the matrix work and the softmax is interleaved with the
// matrix products (the scheduling ideas of the FlashAttention-3 article,
// ybx.com, "FA3 innovations"), here with gfx950 means.
//
// Work decomposition
//   * one workgroup = 4 wavefronts = BM = 128 query rows of one (b, h);
//     each wavefront owns 32 rows.  Two workgroups share a CU.
//   * K and V tiles of BN keys stream HBM -> LDS by buffer loads that write
//     LDS directly (no register staging); out-of-range keys read as zero.
//     Two slots each: tile t+1 is in flight while tile t is multiplied.
//     One barrier per tile.
//   * scores are computed transposed, S^T = K Q^T, on
//     v_mfma_f32_32x32x16_bf16 (A = 32 keys x 16 dims from LDS, B = the Q
//     fragment held in registers).  A lane then holds ONE query and 16 of a
//     block's 32 keys: the row max is in-lane plus one lane^32 exchange, the
//     row sum needs no exchange until the end.
//   * the output is computed transposed too, O^T += V^T P^T: B = the lane's
//     own probabilities in bf16 (no data movement between lanes), A = V^T read
//     with the transposing LDS load ds_read_b64_tr_b16 from a row-major
//     [key][dim] tile.  P lines up with V because K rows sit in LDS with bits
//     2 and 3 of the key index swapped inside each 32-key block, which makes
//     the 8 keys a lane holds for each 16-key step consecutive.
//   * two workgroups share each CU (one wavefront of each per SIMD) and are
//     not coupled by barriers, so one wavefront's softmax overlaps the other's
//     matrix-core work.  The tile loop body is branch-free apart from the
//     rare wave-uniform rescale (a tile no row of the wavefront can see is
//     simply masked to zero weight), which keeps the accumulators in place:
//     no register copies at control-flow joins.
//   * the running max is only raised when a row's new maximum exceeds it by
//     more than kSlack (base-2 units); otherwise probabilities are taken
//     against the old reference (bounded by 2^kSlack), which skips most
//     rescales of the accumulator.  The result is the same exact quantity.
//   * LDS tiles are XOR-swizzled on 16-byte chunks (the buffer loads fetch
//     the permuted source chunk per lane) so the MFMA operand reads are free
//     of bank conflicts.
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
constexpr float kSlack = 8.0f;

// LDS row of key `r` of a K tile: bits 2 and 3 swapped (an involution).
__device__ __forceinline__ int key_slot(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// 16-byte-chunk XOR swizzles of the K and V tiles (row = LDS row).
template <int D>
__device__ __forceinline__ int swz_k(int row) {
  if constexpr (D == 128) return row & 15;
  else return ((row & 3) << 1) ^ ((row >> 2) & 7);
}
template <int D>
__device__ __forceinline__ int swz_v(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) + ((row >> 2) & 3);
  else return ((row & 3) << 1) ^ ((row >> 2) & 7);
}

template <int D, int BN>
__global__ __launch_bounds__(kThreads, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int KCH = D / 8;                      // 16-byte chunks per row
  constexpr int TILE = BN * D;                    // bf16 per K or V tile
  constexpr int NBLK = TILE * 2 / 1024;           // 1 KB load blocks per tile
  constexpr int BPW = NBLK / (kThreads / 64);     // blocks per wavefront
  constexpr int NKB = BN / 32;                    // 32-key blocks per tile
  constexpr int NDB = D / 32;                     // 32-dim blocks of the output
  constexpr int NQK = D / 16;                     // k-steps of q k^T
  static_assert(NBLK % 4 == 0, "tile must split into whole 1 KB blocks per wavefront");

  __shared__ __attribute__((aligned(1024))) uint16_t sK[2][TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t sV[2][TILE];

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

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const uint16_t* kh = a.k + kv_base * D;
  const uint16_t* vh = a.v + kv_base * D;

  const int qw0 = r0 + wave * 32;               // first row of this wavefront
  const int qw1 = min(qw0 + 31, a.Sq - 1);      // last valid row
  const int qi = qw0 + l32;                     // this lane's row
  const bool q_ok = qi < a.Sq;
  const int pos = qi + off;                     // key position aligned with the row
  const int plo = qw0 + off, phi = qw1 + off;

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

  // ---- tile loads: per-lane source offsets are the same for every tile ----
  uint32_t koff[BPW], voff[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int p = (i * (kThreads / 64) + wave) * 64 + lane;  // 16-byte slot in the tile
    const int row = p / KCH, pch = p % KCH;
    koff[i] = (uint32_t)((key_slot(row) * D + (pch ^ swz_k<D>(row)) * 8) * 2);
    voff[i] = (uint32_t)((row * D + (pch ^ swz_v<D>(row)) * 8) * 2);
  }
  const uint32_t sK0 = lds_addr(&sK[0][0]), sV0 = lds_addr(&sV[0][0]);
  auto issue_k = [&](int tile) {
    const int kt = tile * BN;
    const auto rs = make_rsrc(kh + (size_t)kt * D, (uint32_t)(min(BN, a.Sk - kt) * D * 2));
    const uint32_t dst = sK0 + (tile & 1) * (TILE * 2);
#pragma unroll
    for (int i = 0; i < BPW; ++i) dma16(rs, koff[i], dst + (i * (kThreads / 64) + wave) * 1024);
  };
  auto issue_v = [&](int tile) {
    const int kt = tile * BN;
    const auto rs = make_rsrc(vh + (size_t)kt * D, (uint32_t)(min(BN, a.Sk - kt) * D * 2));
    const uint32_t dst = sV0 + (tile & 1) * (TILE * 2);
#pragma unroll
    for (int i = 0; i < BPW; ++i) dma16(rs, voff[i], dst + (i * (kThreads / 64) + wave) * 1024);
  };

  // does every row of this wavefront see every key of tile t?
  auto tile_full = [&](int tile) {
    const int kt0 = tile * BN, kt1 = kt0 + BN - 1;
    bool full = kt1 < a.Sk;
    if (a.causal) full = full && (kt1 <= plo);
    if (w >= 0) full = full && (kt0 >= phi - w) && (kt1 <= plo + w);
    return full;
  };

  // Lane-constant byte offsets of the MFMA operand reads inside one LDS slot.
  // The swizzles only depend on row bits that do not change between 32-key
  // blocks, so block / step offsets become immediates of the ds_read.
  uint32_t ka[NQK];
#pragma unroll
  for (int t = 0; t < NQK; ++t)
    ka[t] = (uint32_t)(l32 * D * 2 + (((2 * t + hh) ^ swz_k<D>(l32)) * 16));
  const int vr0 = 8 * hh + ((lane & 15) >> 2);
  const int vcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  uint32_t va[2][2][NDB];
#pragma unroll
  for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int row = 16 * s2 + vr0 + 4 * r2, col = 32 * db + vcol;
        va[s2][r2][db] = (uint32_t)(row * D * 2 + (((col >> 3) ^ swz_v<D>(row)) * 16) + (col & 7) * 2);
      }

  auto qk = [&](int slot, f32x16* st) {
    const char* kb_base = (const char*)&sK[0][0] + slot * (TILE * 2);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) st[kb] = f32x16{};
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 kf = *(const bf16x8*)(kb_base + ka[t] + kb * 32 * D * 2);
        st[kb] = mfma32(kf, qf[t], st[kb]);
      }
    }
    // issue order: NQK reads, then read/MFMA pairs, then the remaining MFMAs,
    // so every MFMA's operand was requested NQK reads earlier
    __builtin_amdgcn_sched_group_barrier(0x100, NQK, 0);
#pragma unroll
    for (int i = 0; i < NQK * NKB - NQK; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NQK, 0);
  };

  // ---- main loop ----------------------------------------------------------
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m_run = kNegInf;  // reference max of c2 * score (base-2 units)
  float l_run = 0.f;      // this lane's part of the running sum (its 16 keys per block)
  const float c2 = a.c2;
  // keys visible to this lane's row form [key_lo, key_hi] (empty if hi < lo)
  int key_lo = 0, key_hi = a.Sk - 1;
  if (a.causal) key_hi = min(key_hi, pos);
  if (w >= 0) {
    key_lo = max(key_lo, pos - w);
    key_hi = min(key_hi, pos + w);
  }

  // softmax of one tile's scores (in place -> probabilities) and O += V^T P^T
  auto softmax_pv = [&](int slot, int tile, f32x16* st) {
    const int kt0 = tile * BN;
    if (!tile_full(tile)) {
      // accumulator r of block kb holds key kt0 + 8hh + c with c = 32kb + 16(r/8) + r%8
      const int lo = key_lo - kt0 - 8 * hh, hi = key_hi - kt0 - 8 * hh;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int c = kb * 32 + 16 * (r >> 3) + (r & 7);
          st[kb][r] = ((c >= lo) & (c <= hi)) ? st[kb][r] : kNegInf;
        }
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[kb][r]);
    mx = fmaxf(mx, xor_shfl(mx, 32)) * c2;
    if (__any(mx > m_run + kSlack)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    float rs = 0.f;
    bf16x8 pf[NKB][2];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(st[kb][r], c2, -m_use));
        rs += p;
        pf[kb][r >> 3][r & 7] = (__bf16)p;
      }
    l_run += rs;

    // O^T += V^T P^T; the V^T operand for (db, kb, s) is two transposing
    // reads of keys 32kb + 16s + 8hh + [0..3] and [4..7], dims 32db + l32.
    const char* vb = (const char*)&sV[0][0] + slot * (TILE * 2);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char* p0 = vb + kb * 32 * D * 2;
          const s16x4 lo4 = lds_read_tr16((const uint16_t*)(p0 + va[s2][0][db]));
          const s16x4 hi4 = lds_read_tr16((const uint16_t*)(p0 + va[s2][1][db]));
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = mfma32(vf, pf[kb][s2], oacc[db]);
        }
      }
    }
  };

  // K(t) and V(t) land in slot t&1; the loads of tile t+1 are issued as soon
  // as every wavefront is done with tile t-1 (the barrier), so they fly while
  // tile t is multiplied.
  if (t_begin < t_end) {
    issue_k(t_begin);
    issue_v(t_begin);
  }
  for (int tile = t_begin; tile < t_end; ++tile) {
    wait_vmcnt<0>();
    __syncthreads();
    if (tile + 1 < t_end) {
      issue_k(tile + 1);
      issue_v(tile + 1);
    }
    {
      // a tile no row of this wavefront can see is masked to zero weight
      f32x16 st[NKB];
      qk(tile & 1, st);
      softmax_pv(tile & 1, tile, st);
    }
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
    hipLaunchKernelGGL((fwd_bf16_kernel<64, 64>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace ea
