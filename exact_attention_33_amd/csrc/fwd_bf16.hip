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
//   * one workgroup = NW = 8 wavefronts = BM = 256 query rows of one (b, h)
//     (4 wavefronts, 128 rows, for a sliding window at D = 64); each
//     wavefront owns 32 rows.  Every K/V tile written to LDS is read by
//     eight wavefronts, which halves the LDS write traffic and the K/V loads
//     per query row compared with 128-row workgroups.  D = 128: one workgroup
//     per CU (two wavefronts per SIMD); D = 64: two (four per SIMD).
//   * K and V tiles of BN keys (128 at D = 128, 64 at D = 64) stream HBM ->
//     LDS by buffer loads that write LDS directly (no register staging);
//     out-of-range keys read as zero.  Two slots each: tile t+1 is in flight
//     while tile t is multiplied.  One barrier per tile.  (Three slots were
//     measured slower; 128-key tiles at D = 64 need registers that cost a
//     workgroup per CU.)
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
//   * a band (sliding window without a causal mask) is dispatched with a
//     head's query tiles back to back, odd tiles walking their K/V tiles
//     downwards, so two neighbouring query tiles read the K/V they share at
//     about the same time and HBM delivers it once.
//   * two or more wavefronts share each SIMD, so one wavefront's softmax
//     overlaps another's matrix-core work.  Apart from the rare wave-uniform
//     rescale, the only
//     branch in the tile loop skips the matrix work of a tile no row of the
//     wavefront can see (past the causal diagonal, outside the window); the
//     accumulators keep one register home across it.
//   * the running max is only raised when a row's new maximum exceeds it by
//     more than kSlack (base-2 units); otherwise probabilities are taken
//     against the old reference (bounded by 2^kSlack), which skips most
//     rescales of the accumulator.  The result is the same exact quantity.
//   * LDS layout (D = 128): rows are padded (K: 272 bytes, V: 320 bytes) so
//     the MFMA operand reads are free of bank conflicts and every read
//     address is one lane base plus an immediate offset.  D = 64 tiles are
//     dense and XOR-swizzled on 16-byte chunks instead (the buffer loads
//     fetch the permuted source chunk per lane).
//   * the row max needs one exchange between lanes l and l^32
//     (v_permlane32_swap); no LDS traffic.
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

template <int D, int BN, int NW>
__global__ __launch_bounds__(64 * NW, 2) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int BM = 32 * NW;                     // query rows per workgroup
  constexpr int KCH = D / 8;                      // 16-byte chunks per row
  constexpr int NKB = BN / 32;                    // 32-key blocks per tile
  constexpr int NDB = D / 32;                     // 32-dim blocks of the output
  constexpr int NQK = D / 16;                     // k-steps of q k^T

  // padded rows (D = 128): operand addresses are a lane base plus immediates
  constexpr bool PAD = (D == 128);
  constexpr int KS = PAD ? D * 2 + 16 : D * 2;   // LDS row strides (bytes)
  constexpr int VS = PAD ? D * 2 + 64 : D * 2;
  constexpr int KSLOT = BN * KS, VSLOT = BN * VS;
  constexpr int NB = (KSLOT + VSLOT) / 1024;     // 1 KB DMA blocks per (K, V) tile pair
  constexpr int NBW = (NB + NW - 1) / NW;        // per wavefront (at most)
  static_assert(KSLOT % 1024 == 0 && VSLOT % 1024 == 0, "whole blocks");
  __shared__ __attribute__((aligned(1024))) char sK[2 * KSLOT];
  __shared__ __attribute__((aligned(1024))) char sV[2 * VSLOT];

  // ---- which (b, h, query tile) this workgroup computes -----------------
  const int BH = a.B * a.Hq;
  int bh, rank;
  if (a.xcd_heads > 0) {
    // Blocks are dispatched round-robin over the 8 XCDs; give each XCD a
    // contiguous set of heads so a head's K/V stays in one L2.
    const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    if (a.window >= 0 && !a.causal) {
      // a band: a head's query tiles back to back, so neighbouring tiles,
      // which share K/V, run at the same time (see the tile order below)
      bh = xcd * a.xcd_heads + slot / a.n_qtiles;
      rank = slot % a.n_qtiles;
    } else {
      bh = xcd * a.xcd_heads + slot % a.xcd_heads;
      rank = slot / a.xcd_heads;
    }
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

  const int r0 = qtile * BM;
  const int r1 = min(r0 + BM, a.Sq) - 1;
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
  // block bb < KSLOT/1024 of a tile pair is a K block, the rest V blocks;
  // wavefront w issues blocks w, w+4, ...
  uint32_t doff[NBW], ddst[NBW];
  bool disk[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int bb = i * NW + wave;
    disk[i] = bb < KSLOT / 1024;
    if (disk[i]) {
      const int p = bb * 64 + lane;
      if constexpr (PAD) {
        const int row = p / (KS / 16), u = p % (KS / 16);
        doff[i] = (u < 16) ? (uint32_t)((key_slot(row) * D + u * 8) * 2) : 0x7ffffff0u;
      } else {
        const int row = p / KCH, pch = p % KCH;
        doff[i] = (uint32_t)((key_slot(row) * D + (pch ^ swz_k<D>(row)) * 8) * 2);
      }
      ddst[i] = (uint32_t)(bb * 1024);
    } else {
      const int vb = bb - KSLOT / 1024;
      const int p = vb * 64 + lane;
      if constexpr (PAD) {
        const int row = p / (VS / 16), u = p % (VS / 16);
        doff[i] = (u < 16 && row < BN) ? (uint32_t)((row * D + u * 8) * 2) : 0x7ffffff0u;
      } else {
        const int row = p / KCH, pch = p % KCH;
        doff[i] = (uint32_t)((row * D + (pch ^ swz_v<D>(row)) * 8) * 2);
      }
      ddst[i] = (uint32_t)(vb * 1024);
    }
  }
  const int nbw = (NB - wave + NW - 1) / NW;   // blocks this wavefront issues
  const uint32_t sK0 = lds_addr(sK), sV0 = lds_addr(sV);
  auto issue = [&](int tile, int slot) {
    const int kt = tile * BN;
    const uint32_t bytes = (uint32_t)(min(BN, a.Sk - kt) * D * 2);
    const auto rk = make_rsrc(kh + (size_t)kt * D, bytes);
    const auto rv = make_rsrc(vh + (size_t)kt * D, bytes);
    const uint32_t kdst = sK0 + slot * KSLOT, vdst = sV0 + slot * VSLOT;
#pragma unroll
    for (int i = 0; i < NBW - 1; ++i) dma16(disk[i] ? rk : rv, doff[i], (disk[i] ? kdst : vdst) + ddst[i]);
    if (NB % NW == 0 || nbw == NBW)
      dma16(disk[NBW - 1] ? rk : rv, doff[NBW - 1], (disk[NBW - 1] ? kdst : vdst) + ddst[NBW - 1]);
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
  uint32_t ka[PAD ? 1 : NQK];
  if constexpr (PAD) {
    ka[0] = (uint32_t)(l32 * KS + 16 * hh);
  } else {
#pragma unroll
    for (int t = 0; t < NQK; ++t)
      ka[t] = (uint32_t)(l32 * D * 2 + (((2 * t + hh) ^ swz_k<D>(l32)) * 16));
  }
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
        if constexpr (PAD)
          va[s2][r2][db] = (uint32_t)(row * VS + col * 2);
        else
          va[s2][r2][db] = (uint32_t)(row * D * 2 + (((col >> 3) ^ swz_v<D>(row)) * 16) + (col & 7) * 2);
      }

  auto qk = [&](int slot, f32x16* st) {
    const char* kb_base = sK + slot * KSLOT;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) st[kb] = f32x16{};
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8 kf = PAD ? *(const bf16x8*)(kb_base + ka[0] + kb * 32 * KS + 32 * t)
                              : *(const bf16x8*)(kb_base + ka[PAD ? 0 : t] + kb * 32 * D * 2);
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
    mx = max_swap32(mx) * c2;
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
    const char* vb = sV + slot * VSLOT;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const char* p0 = vb + kb * 32 * (PAD ? VS : D * 2);
          const s16x4 lo4 = lds_read_tr16((const uint16_t*)(p0 + va[s2][0][db]));
          const s16x4 hi4 = lds_read_tr16((const uint16_t*)(p0 + va[s2][1][db]));
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = mfma32(vf, pf[kb][s2], oacc[db]);
        }
      }
    }
  };

  // The K/V of step i land in slot i&1; the loads of step i+1 are issued as
  // soon as every wavefront is done with step i-1 (the barrier), so they fly
  // while step i is multiplied.
  // A band (window, no causal mask): odd query tiles walk their K/V tiles
  // downwards.  Query tiles r and r + 1 share their K/V tiles at the edge
  // between them; with the alternating order both reach those tiles at the
  // same step of their walk, one dispatch apart, so the second read finds
  // them in L2 (HBM reads of the window-encoder shape: 402 MB -> 304 MB,
  // the size of q, k and v).
  const bool down = (w >= 0) && !a.causal && (qtile & 1);
  const int n_t = t_end - t_begin;
  auto tile_at = [&](int i) { return down ? t_end - 1 - i : t_begin + i; };
  if (n_t > 0) issue(tile_at(0), 0);
  for (int i = 0; i < n_t; ++i) {
    const int tile = tile_at(i);
    wait_vmcnt<0>();
    __syncthreads();
    if (i + 1 < n_t) issue(tile_at(i + 1), (i + 1) & 1);
    // skip the matrix work of a tile no row of this wavefront can see
    const int kt0 = tile * BN, kt1 = kt0 + BN - 1;
    bool any = kt0 < a.Sk;
    if (a.causal) any = any && (kt0 <= phi);
    if (w >= 0) any = any && (kt0 <= phi + w) && (kt1 >= plo - w);
    if (any) {
      f32x16 st[NKB];
      qk(i & 1, st);
      softmax_pv(i & 1, tile, st);
    }
  }

  // ---- epilogue: normalise, round once to bf16, write o and lse ----------
  const float l_tot = sum_swap32(l_run);
  const float inv = (l_tot > 0.f) ? 1.f / l_tot : 0.f;
  uint16_t* orow = a.o + (q_base + (q_ok ? qi : 0)) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_row32_bf16(orow + db * 32, oacc[db], inv, hh, q_ok);
  if (q_ok && a.lse != nullptr && hh == 0)
    a.lse[q_base + qi] = (l_tot > 0.f) ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
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
  // 8 wavefronts of 32 rows; 4 for a sliding window at D = 64, where a
  // workgroup's few tiles make its start and end weigh more and four
  // resident workgroups per CU cover them (measured 104.7 against 106.6 us
  // on the window-encoder shape; 3 % slower without a window)
  const bool narrow = (s.D == 64) && (s.window >= 0);
  const int bm = narrow ? 128 : 256;
  a.n_qtiles = (s.Sq + bm - 1) / bm;
  const int BH = s.B * s.Hq;
  const int64_t nblocks = (int64_t)a.n_qtiles * BH;
  a.xcd_heads = (BH % 8 == 0) ? BH / 8 : 0;
  dim3 grid((unsigned)nblocks), block(bm / 32 * 64);
  if (s.D == 128)
    hipLaunchKernelGGL((fwd_bf16_kernel<128, 128, 8>), grid, block, 0, stream, a);
  else if (narrow)
    hipLaunchKernelGGL((fwd_bf16_kernel<64, 64, 4>), grid, block, 0, stream, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<64, 64, 8>), grid, block, 0, stream, a);
  return hipGetLastError();
}

}  // namespace ea
