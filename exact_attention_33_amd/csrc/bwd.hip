// Backward of exact attention for gfx950: the gradients dq, dk, dv of
// sum(dout * o) with o = softmax(scale * q k^T) v, recomputing the
// probabilities from the forward's log-sum-exp instead of storing them (the
// pages name training as a use of the fused method -- FlashAttention
// explainer, "Overview"; FlashAttention-3 article, "Benefits of
// FlashAttention-3" -- and the N x N matrix is never written in this
// direction either).
//
// With s = scale q k^T, P = exp(s - lse), dP = dout v^T,
// delta_i = sum_d dout[i,d] o[i,d] and dS = P * (dP - delta):
//   dv = P^T dout,  dk = scale dS^T q,  dq = scale dS k.
//
// Two kernels, launched in this order on one stream:
//   * bwd_dq_kernel: one workgroup = 8 wavefronts x 32 query rows of one
//     (b, h), causal tiles heaviest first.  q and dout stay in registers;
//     K/V stages of 128 keys (four 32-key blocks per barrier, each of the 8
//     wavefronts loading one K or V tile) stream through LDS, shared by the
//     8 wavefronts.  Per tile and wavefront: S^T = K
//     q^T and dP^T = V dout^T (A = 32 keys from LDS, B = the wavefront's 32
//     queries in registers), so a lane holds one query and its lse / delta
//     are lane scalars; then dq^T += K^T dS^T with K^T read by the
//     transposing LDS load.  A 32-key block no row of the wavefront sees is
//     skipped.  It first computes delta for its rows and writes it for the
//     second kernel.
//   * bwd_dkdv_kernel: one workgroup = 4 wavefronts x 32 keys of one
//     (b, kv head).  k and v stay in registers; q / dout tiles of 32 rows of
//     every query head of the GQA group stream through LDS (with their lse
//     and delta).  Per tile: S = q k^T and dP = dout v^T (A = 32 query rows
//     from LDS, B = the wavefront's keys), a lane holding one key; then
//     dv^T += dout^T P and dk^T += q^T dS.  The group's query heads are summed
//     in registers, so no atomics are needed.
// Both kernels run two wavefronts per SIMD (one dq workgroup or two dk/dv
// workgroups per CU), so one wavefront's softmax-side vector work overlaps
// the other's matrix work.
// The A-operand rows of S / S^T and dP / dP^T are read with bits 2 and 3 of
// the row index swapped; the 8 values a lane then holds for each 16-row
// MFMA step are consecutive rows, which is the B-operand layout of the
// following product (no data movement between lanes).
#include "common.h"
#include "kernels.h"

namespace ea {
namespace {

constexpr int kThreadsB = 256;      // dk/dv kernel: 4 wavefronts x 32 keys
constexpr int kThreadsDq = 512;     // dq kernel: 8 wavefronts x 32 query rows
constexpr int kRowsDq = kThreadsDq / 2;
constexpr float kBwdLog2e = 1.4426950408889634f;

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;
  int B, Hq, Hkv, Sq, Sk;
  int causal, window;
  float c2;     // scale * log2(e)
  float scale;
};

// row index with bits 2 and 3 swapped (an involution)
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// LDS geometry of a 32-row bf16 tile with padded rows: conflict-free (or
// 2-way at worst) for both the 16-byte operand reads and the transposing
// reads, and every read address is a lane base plus an immediate.
template <int D>
struct TileGeo {
  static constexpr int RS = (D == 128) ? 304 : 144;                 // row stride, bytes
  static constexpr int RU = RS / 16;                                  // 16-byte units per row
  static constexpr int BYTES = (32 * RS + 1023) / 1024 * 1024;        // whole 1 KB blocks
  static constexpr int BLK = BYTES / 1024;
};

// Per-lane source offset of unit p of a padded 32-row tile (out of range for
// padding units: the buffer load then returns zero).
template <int D>
__device__ __forceinline__ uint32_t tile_src(int p) {
  using G = TileGeo<D>;
  const int row = p / G::RU, u = p % G::RU;
  return (u < D / 8 && row < 32) ? (uint32_t)((row * D + u * 8) * 2) : 0x7ffffff0u;
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreadsDq, 2) void bwd_dq_kernel(BwdArgs a) {
  using G = TileGeo<D>;
  constexpr int NQK = D / 16;    // k-steps over dims
  constexpr int NDB = D / 32;    // 32-dim blocks of dq^T
  // a stage holds 128 keys as eight padded 32-row tiles: K0..K3 | V0..V3;
  // wavefront w loads tile w
  constexpr int NJ = 4;                       // 32-key blocks per stage
  __shared__ __attribute__((aligned(1024))) char sT[2][2 * NJ * G::BYTES];

  const int BH = a.B * a.Hq;
  // causal: the heaviest query tiles (most keys) first, so they do not
  // start last and set the kernel's tail
  const int nq = (a.Sq + kRowsDq - 1) / kRowsDq;
  const int bh = blockIdx.x % BH, rank = blockIdx.x / BH;
  const int qtile = a.causal ? nq - 1 - rank : rank;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int g = h / (a.Hq / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  const int off = a.Sk - a.Sq;
  const int w = a.window;

  const int r0 = qtile * kRowsDq;
  const int r1 = min(r0 + kRowsDq, a.Sq) - 1;
  int kv_lo = 0, kv_hi = a.Sk;
  if (a.causal) kv_hi = min(kv_hi, r1 + off + 1);
  if (w >= 0) {
    kv_lo = max(kv_lo, r0 + off - w);
    kv_hi = min(kv_hi, r1 + off + w + 1);
  }
  const int t_begin = max(kv_lo, 0) / (32 * NJ);
  const int t_end = (kv_hi > kv_lo) ? (kv_hi + 32 * NJ - 1) / (32 * NJ) : t_begin;

  const size_t q_base = ((size_t)b * a.Hq + h) * (size_t)a.Sq;
  const size_t kv_base = ((size_t)b * a.Hkv + g) * (size_t)a.Sk;
  const uint16_t* kh = a.k + kv_base * D;
  const uint16_t* vh = a.v + kv_base * D;

  const int qw0 = r0 + wave * 32;
  const int qi = qw0 + l32;
  const bool q_ok = qi < a.Sq;
  const int pos = qi + off;
  const int plo = qw0 + off, phi = min(qw0 + 31, a.Sq - 1) + off;   // this wavefront's positions

  // q and dout of this lane's row (B operands), delta from o and dout
  bf16x8 qf[NQK], df[NQK];
  float dpart = 0.f;
  {
    const size_t row = (q_base + (q_ok ? qi : 0)) * D;
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
      const u32x4 zq = {0, 0, 0, 0};
      const u32x4 rq = q_ok ? *(const u32x4*)(a.q + row + 16 * t + 8 * hh) : zq;
      const u32x4 rd = q_ok ? *(const u32x4*)(a.dout + row + 16 * t + 8 * hh) : zq;
      const u32x4 ro = q_ok ? *(const u32x4*)(a.o + row + 16 * t + 8 * hh) : zq;
      qf[t] = __builtin_bit_cast(bf16x8, rq);
      df[t] = __builtin_bit_cast(bf16x8, rd);
      const bf16x8 of = __builtin_bit_cast(bf16x8, ro);
#pragma unroll
      for (int j = 0; j < 8; ++j) dpart += (float)df[t][j] * (float)of[j];
    }
  }
  const float delta = sum_swap32(dpart);
  float lse2 = q_ok ? a.lse[q_base + qi] : 0.f;
  lse2 = (lse2 == kNegInf) ? __builtin_inff() : lse2 * kBwdLog2e;
  if (q_ok && hh == 0) a.delta[q_base + qi] = delta;

  // keys visible to this lane's row: [key_lo, key_hi]
  int key_lo = 0, key_hi = a.Sk - 1;
  if (a.causal) key_hi = min(key_hi, pos);
  if (w >= 0) {
    key_lo = max(key_lo, pos - w);
    key_hi = min(key_hi, pos + w);
  }
  if (!q_ok) key_hi = -1;

  // tile loads: wavefront w fills tile w of the stage (K0..K3, V0..V3)
  uint32_t doff[G::BLK];
#pragma unroll
  for (int i = 0; i < G::BLK; ++i) doff[i] = tile_src<D>(i * 64 + lane);
  const uint16_t* src_base = (wave < NJ) ? kh : vh;
  const int src_off = (wave % NJ) * 32;
  const uint32_t sT0 = lds_addr(&sT[0][0]);
  auto issue = [&](int tile, int st) {
    const int kt = tile * 32 * NJ + src_off;
    const int rows = max(0, min(32, a.Sk - kt));
    const auto rs = make_rsrc(src_base + (size_t)(rows > 0 ? kt : 0) * D, (uint32_t)(rows * D * 2));
    const uint32_t base = sT0 + st * (2 * NJ * G::BYTES) + wave * G::BYTES;
#pragma unroll
    for (int i = 0; i < G::BLK; ++i) dma16(rs, doff[i], base + i * 1024);
  };

  // lane bases of the operand reads inside one tile
  const uint32_t a_row = (uint32_t)(swap23(l32) * G::RS + 16 * hh);           // 16-byte A reads
  const int tr_row = 8 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t tr_base = (uint32_t)(tr_row * G::RS + tr_col * 2);           // transposing reads

  f32x16 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x16{};
  const float c2 = a.c2;

  if (t_begin < t_end) issue(t_begin, 0);
  for (int tile = t_begin; tile < t_end; ++tile) {
    const int st = (tile - t_begin) & 1;
    wait_vmcnt<0>();
    __syncthreads();
    if (tile + 1 < t_end) issue(tile + 1, st ^ 1);
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
    // skip a 32-key block no row of this wavefront can see
    const int kb0 = tile * 32 * NJ + 32 * j;
    bool any = kb0 < a.Sk;
    if (a.causal) any = any && (kb0 <= phi);
    if (w >= 0) any = any && (kb0 <= phi + w) && (kb0 + 31 >= plo - w);
    if (!any) continue;
    const char* kb = &sT[st][j * G::BYTES];
    const char* vb = &sT[st][(NJ + j) * G::BYTES];

    // S^T = K q^T, dP^T = V dout^T (32 keys x 32 queries each)
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
      const bf16x8 ka = *(const bf16x8*)(kb + a_row + 32 * t);
      const bf16x8 va = *(const bf16x8*)(vb + a_row + 32 * t);
      s = mfma32(ka, qf[t], s);
      dp = mfma32(va, df[t], dp);
    }
    // element r holds key kt0 + 16*(r/8) + 8*hh + r%8 of this lane's query
    const int kt0 = tile * 32 * NJ + 32 * j;
    const int lo = key_lo - kt0 - 8 * hh, hi = key_hi - kt0 - 8 * hh;
    bf16x8 dsb[2];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int c = 16 * (r >> 3) + (r & 7);
      const bool vis = (c >= lo) & (c <= hi);
      const float p = vis ? fast_exp2(__builtin_fmaf(s[r], c2, -lse2)) : 0.f;
      dsb[r >> 3][r & 7] = (__bf16)(p * (dp[r] - delta));
    }
    // dq^T += K^T dS^T
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const char* p0 = kb + tr_base + (16 * s2) * G::RS + 64 * db;
        const s16x4 lo4 = lds_read_tr16((const uint16_t*)p0);
        const s16x4 hi4 = lds_read_tr16((const uint16_t*)(p0 + 4 * G::RS));
        const bf16x8 kt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = mfma32(kt, dsb[s2], acc[db]);
      }
    }
  }

  uint16_t* orow = a.dq + (q_base + (q_ok ? qi : 0)) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) store_row32_bf16(orow + db * 32, acc[db], a.scale, hh, q_ok);
}

// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreadsB, 2) void bwd_dkdv_kernel(BwdArgs a) {
  using G = TileGeo<D>;
  constexpr int NQK = D / 16;
  constexpr int NDB = D / 32;
  constexpr int NB2 = 2 * G::BLK;                 // blocks of a (q, dout) stage
  constexpr int NBW = (NB2 + 3) / 4;
  constexpr int STAGE = 2 * G::BYTES + 2048;      // q | dout | lse (1 KB) | delta (1 KB)
  __shared__ __attribute__((aligned(1024))) char sT[2][STAGE];

  const int BK = a.B * a.Hkv;
  const int bg = blockIdx.x % BK, ktile = blockIdx.x / BK;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int GQ = a.Hq / a.Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  const int off = a.Sk - a.Sq;
  const int w = a.window;

  const int k0 = ktile * 128;
  const int k1 = min(k0 + 128, a.Sk) - 1;
  // query rows that see some key of [k0, k1]
  int q_lo = 0, q_hi = a.Sq - 1;
  if (a.causal) q_lo = max(q_lo, k0 - off);
  if (w >= 0) {
    q_lo = max(q_lo, k0 - off - w);
    q_hi = min(q_hi, k1 - off + w);
  }
  const int t_begin = q_lo / 32;
  const int t_end = (q_hi >= q_lo) ? q_hi / 32 + 1 : t_begin;
  const int nt = t_end - t_begin;

  const size_t kv_base = ((size_t)b * a.Hkv + g) * (size_t)a.Sk;
  const int kk = k0 + wave * 32 + l32;          // this lane's key
  const bool k_ok = kk < a.Sk;

  // k and v of this lane's key (B operands)
  bf16x8 kf[NQK], vf[NQK];
  {
    const size_t row = (kv_base + (k_ok ? kk : 0)) * D;
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
      const u32x4 z = {0, 0, 0, 0};
      kf[t] = __builtin_bit_cast(bf16x8, k_ok ? *(const u32x4*)(a.k + row + 16 * t + 8 * hh) : z);
      vf[t] = __builtin_bit_cast(bf16x8, k_ok ? *(const u32x4*)(a.v + row + 16 * t + 8 * hh) : z);
    }
  }
  // query rows that see this lane's key: [row_lo, row_hi]
  int row_lo = 0, row_hi = a.Sq - 1;
  if (a.causal) row_lo = max(row_lo, kk - off);
  if (w >= 0) {
    row_lo = max(row_lo, kk - off - w);
    row_hi = min(row_hi, kk - off + w);
  }
  if (!k_ok) row_hi = -1;

  // Source offsets of this lane's DMA chunks, two 16-bit offsets per
  // register (a tile is at most 8 KB; 0xffff lies past every tile's buffer
  // range and reads zero): at 256 VGPRs a register more spills, and a
  // spilled offset's reload waits for the stage's own DMA loads.
  uint32_t doffp[(NBW + 1) / 2] = {}, ddst[NBW];
  bool disq[NBW];
#pragma unroll
  for (int i = 0; i < NBW; ++i) {
    const int bb = i * 4 + wave;
    disq[i] = bb < G::BLK;
    const int tb = disq[i] ? bb : bb - G::BLK;
    const uint32_t o = tile_src<D>(tb * 64 + lane);
    doffp[i >> 1] |= (o < 0xffffu ? o : 0xffffu) << (16 * (i & 1));
    ddst[i] = (uint32_t)(bb * 1024);
  }
  const uint32_t sT0 = lds_addr(&sT[0][0]);
  // stage `it` of the flattened (query head, query tile) sequence
  auto issue = [&](int it, int st) {
    const int hq = g * GQ + it / nt;
    const int qt = (t_begin + it % nt) * 32;
    const size_t qb = ((size_t)b * a.Hq + hq) * (size_t)a.Sq;
    const uint32_t rows = (uint32_t)min(32, a.Sq - qt);
    const auto rq = make_rsrc(a.q + (qb + qt) * D, rows * D * 2);
    const auto rd = make_rsrc(a.dout + (qb + qt) * D, rows * D * 2);
    const uint32_t base = sT0 + st * STAGE;
#pragma unroll
    for (int i = 0; i < NBW; ++i)
      if (i * 4 + wave < NB2) {
        // unpacked here, at the load (volatile keeps the compiler from
        // hoisting five unpacked registers out of the loop)
        uint32_t o;
        asm volatile("v_bfe_u32 %0, %1, %2, 16" : "=v"(o) : "v"(doffp[i >> 1]), "i"(16 * (i & 1)));
        dma16(disq[i] ? rq : rd, o, base + ddst[i]);
      }
    if (wave == 0) {
      const uint32_t lo = (lane < 8) ? (uint32_t)(lane * 16) : 0x7ffffff0u;
      dma16(make_rsrc(a.lse + qb + qt, rows * 4), lo, base + 2 * G::BYTES);
      dma16(make_rsrc(a.delta + qb + qt, rows * 4), lo, base + 2 * G::BYTES + 1024);
    }
  };

  const uint32_t a_row = (uint32_t)(swap23(l32) * G::RS + 16 * hh);
  const int tr_row = 8 * hh + ((lane & 15) >> 2);
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const uint32_t tr_base = (uint32_t)(tr_row * G::RS + tr_col * 2);

  f32x16 dka[NDB], dva[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dka[i] = f32x16{};
    dva[i] = f32x16{};
  }
  const float c2 = a.c2;
  const int n_it = nt * GQ;

  if (n_it > 0) issue(0, 0);
  for (int it = 0; it < n_it; ++it) {
    const int st = it & 1;
    wait_vmcnt<0>();
    __syncthreads();
    if (it + 1 < n_it) issue(it + 1, st ^ 1);
    const char* qb = &sT[st][0];
    const char* db_ = &sT[st][G::BYTES];
    const float* lse_t = (const float*)&sT[st][2 * G::BYTES];
    const float* del_t = (const float*)&sT[st][2 * G::BYTES + 1024];
    const int qt = (t_begin + it % nt) * 32;

    // S = q k^T and dP = dout v^T (32 queries x 32 keys)
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
      const bf16x8 qa = *(const bf16x8*)(qb + a_row + 32 * t);
      const bf16x8 da = *(const bf16x8*)(db_ + a_row + 32 * t);
      s = mfma32(qa, kf[t], s);
      dp = mfma32(da, vf[t], dp);
    }
    // element r holds query qt + 16*(r/8) + 8*hh + r%8 of this lane's key
    const int lo = row_lo - qt - 8 * hh, hi = row_hi - qt - 8 * hh;
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const f32x4 l0 = *(const f32x4*)(lse_t + 16 * s2 + 8 * hh);
      const f32x4 l1 = *(const f32x4*)(lse_t + 16 * s2 + 8 * hh + 4);
      const f32x4 d0 = *(const f32x4*)(del_t + 16 * s2 + 8 * hh);
      const f32x4 d1 = *(const f32x4*)(del_t + 16 * s2 + 8 * hh + 4);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * s2 + j;
        const int c = 16 * s2 + j;
        const bool vis = (c >= lo) & (c <= hi);
        const float lsev = (j < 4) ? l0[j] : l1[j - 4];
        const float delv = (j < 4) ? d0[j] : d1[j - 4];
        const float p = vis ? fast_exp2(__builtin_fmaf(s[r], c2, -lsev * kBwdLog2e)) : 0.f;
        pb[s2][j] = (__bf16)p;
        dsb[s2][j] = (__bf16)(p * (dp[r] - delv));
      }
    }
    // dv^T += dout^T P, dk^T += q^T dS
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int dbk = 0; dbk < NDB; ++dbk) {
        const uint32_t o0 = tr_base + (16 * s2) * G::RS + 64 * dbk;
        const s16x4 dlo = lds_read_tr16((const uint16_t*)(db_ + o0));
        const s16x4 dhi = lds_read_tr16((const uint16_t*)(db_ + o0 + 4 * G::RS));
        const s16x4 qlo = lds_read_tr16((const uint16_t*)(qb + o0));
        const s16x4 qhi = lds_read_tr16((const uint16_t*)(qb + o0 + 4 * G::RS));
        const bf16x8 dt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 qt8 = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
        dva[dbk] = mfma32(dt, pb[s2], dva[dbk]);
        dka[dbk] = mfma32(qt8, dsb[s2], dka[dbk]);
      }
  }

  // 8-byte stores here: at 256 VGPRs the exchange of the 16-byte store
  // helper costs a register, which spills inside the loop
  if (k_ok) {
    uint16_t* krow = a.dk + (kv_base + kk) * D;
    uint16_t* vrow = a.dv + (kv_base + kk) * D;
#pragma unroll
    for (int dbk = 0; dbk < NDB; ++dbk)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        bf16x4 kv4, vv4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kv4[j] = (__bf16)(dka[dbk][4 * g4 + j] * a.scale);
          vv4[j] = (__bf16)dva[dbk][4 * g4 + j];
        }
        *(bf16x4*)(krow + dbk * 32 + 8 * g4 + 4 * hh) = kv4;
        *(bf16x4*)(vrow + dbk * 32 + 8 * g4 + 4 * hh) = vv4;
      }
  }
}

}  // namespace

hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                      const uint16_t* dout, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                      float* delta, const FwdShape& s, hipStream_t stream) {
  BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.delta = delta;
  a.B = s.B;
  a.Hq = s.Hq;
  a.Hkv = s.Hkv;
  a.Sq = s.Sq;
  a.Sk = s.Sk;
  a.causal = s.causal;
  a.window = s.window;
  a.c2 = s.scale * kBwdLog2e;
  a.scale = s.scale;
  const int64_t nq = (int64_t)((s.Sq + kRowsDq - 1) / kRowsDq) * s.B * s.Hq;
  const int64_t nk = (int64_t)((s.Sk + 127) / 128) * s.B * s.Hkv;
  if (s.D == 128) {
    if (nq > 0) hipLaunchKernelGGL(bwd_dq_kernel<128>, dim3((unsigned)nq), dim3(kThreadsDq), 0, stream, a);
    if (nk > 0) hipLaunchKernelGGL(bwd_dkdv_kernel<128>, dim3((unsigned)nk), dim3(kThreadsB), 0, stream, a);
  } else {
    if (nq > 0) hipLaunchKernelGGL(bwd_dq_kernel<64>, dim3((unsigned)nq), dim3(kThreadsDq), 0, stream, a);
    if (nk > 0) hipLaunchKernelGGL(bwd_dkdv_kernel<64>, dim3((unsigned)nk), dim3(kThreadsB), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace ea
