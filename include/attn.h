/*
 * attn.h -- exact softmax attention on AMD Instinct MI355X (gfx950), C ABI.
 *
 * What is computed (all entry points): for every batch b, query head h and
 * query row i,
 *
 *     s_ij   = scale * <q[b,h,i,:], k[b,g,j,:]>          g = h / (Hq / Hkv)
 *     lse_i  = ln( sum_{j visible} exp(s_ij) )
 *     o_i    = sum_{j visible} exp(s_ij - lse_i) * v[b,g,j,:]
 *
 * i.e. standard attention; the FlashAttention explainer (aiunderstanding.org,
 * "Deep dive" and FAQ) states the tiled fused method returns exactly these
 * values while never writing the score matrix to memory, which is what the
 * kernels behind this header do.  The split-KV decode merges per-chunk
 * partials with the log-sum-exp operator in a tree along the sequence axis
 * (Tree Attention abstract, express24.ir page).
 *
 * Visibility of key j to query i, with c = i + (Sk - Sq) (bottom-right
 * alignment):  [causal == 0 || j <= c]  &&  [window < 0 || |c - j| <= window].
 * A sliding window is local attention -- each token attends only to its
 * neighbours (thread on extending LLM context, point 1).  A row with no
 * visible key gets o = 0 and lse = -inf.
 *
 * Layout: every tensor is dense, row-major, last dimension fastest:
 *     q, o   [B, Hq,  Sq, D]     (decode: [B, Hq, D])
 *     k, v   [B, Hkv, Sk, D]     (decode: the KV cache, same shape)
 *     lse    [B, Hq,  Sq] fp32   (decode: [B, Hq])
 * Device pointers only (memory from hipMalloc or a framework allocator on the
 * current device).  The kernels move whole 16-byte vectors: q, k, v, o, the
 * gradient tensors and the decode workspace must start on a 16-byte
 * boundary, lse and delta on a 4-byte boundary (ATTN_ERR_ARG otherwise).
 * The caller owns every buffer; the library never frees or keeps a caller
 * pointer after the call returns.
 *
 * Execution: every call only enqueues work on `stream` (NULL = the default
 * stream) and returns; there is no host synchronisation.  Arguments are
 * checked on the host first; on any error nothing is enqueued and nothing is
 * written.  No C++ exception crosses this boundary.  Return value: ATTN_OK or
 * one of the codes below; attn_error_string() names it.
 */
#ifndef EXACT_ATTENTION_ATTN_H
#define EXACT_ATTENTION_ATTN_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = 1,      /* a required pointer is NULL                                  */
  ATTN_ERR_SHAPE = 2,     /* a size is negative, or too large for the kernels' indexing
                             or for one launch (grid blocks x threads must stay < 2^32) */
  ATTN_ERR_GQA = 3,       /* Hkv < 1 while Hq > 0, or Hq % Hkv != 0                      */
  ATTN_ERR_HEADDIM = 4,   /* D is not 64 or 128                                          */
  ATTN_ERR_SPLITS = 5,    /* num_splits < 1, or num_splits > max(Sk, 1)                  */
  ATTN_ERR_WINDOW = 6,    /* window < -1                                                 */
  ATTN_ERR_WORKSPACE = 7, /* workspace NULL or smaller than attn_decode_workspace_bytes */
  ATTN_ERR_HIP = 8,       /* the HIP runtime reported an error (launch, allocation)      */
  ATTN_ERR_ARG = 9        /* causal not 0/1, scale not finite and > 0, or a pointer     */
                          /* misaligned (see "Layout" above)                           */
} attn_status;

/*
 * Prefill forward pass, bf16 q/k/v/o, fp32 accumulation and softmax.
 *
 *   q, k, v, o : bf16 device tensors in the layout above (k, v may be NULL
 *                when Sk == 0; nothing is read or written when B*Hq*Sq == 0).
 *   lse        : fp32 [B, Hq, Sq], or NULL to skip it.
 *   causal     : 0 or 1.   window: -1 for none, else the half width w >= 0.
 *   scale      : finite, > 0 (usually 1/sqrt(D)).
 *   D          : 64 or 128.   Hq % Hkv == 0.
 * o is rounded once, round-to-nearest-even, from fp32.  One kernel launch;
 * the Sq x Sk score matrix never leaves the chip.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int D,
             int causal, int window, float scale, hipStream_t stream);

/*
 * The same computation for fp32 q/k/v/o; arithmetic stays in fp32 (nothing
 * is rounded to bf16).  Same arguments and errors as attn_fwd.
 */
int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int D,
                 int causal, int window, float scale, hipStream_t stream);

/*
 * Prefill on fp8 inputs: q, k, v are OCP FP8 E4M3 ("e4m3fn") byte codes with
 * one descale factor per tensor; the result is the attention of the real
 * inputs decode(code) * descale, with o in bf16 and lse in fp32 (natural log,
 * scale and descales included).  FlashAttention-3 takes attention to
 * low-precision FP8 (FlashAttention explainer, aiunderstanding.org, "The
 * future of FlashAttention" and the FAQ entry on FlashAttention-3;
 * FlashAttention-3 article, ybx.com, "FA3 innovations" point 3); the pages fix
 * no format or scaling, these are readings.
 *
 *   q8      : uint8 codes [B, Hq, Sq, D].   k8, v8: uint8 codes [B, Hkv, Sk, D].
 *   o       : bf16 [B, Hq, Sq, D].           lse: fp32 [B, Hq, Sq] or NULL.
 *   D       : 64 or 128 (ATTN_ERR_HEADDIM otherwise), as attn_fwd.
 *   q_descale, k_descale, v_descale: finite and > 0 (ATTN_ERR_ARG otherwise).
 *   Other arguments and errors as attn_fwd.
 * The probabilities are rounded to e4m3 (round to nearest even) before the
 * p.v product on the fp8 matrix cores; scores, softmax and accumulation are
 * fp32; o is rounded once to bf16.
 */
int attn_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int D,
                 int causal, int window, float scale,
                 float q_descale, float k_descale, float v_descale, hipStream_t stream);

/*
 * Backward of attn_fwd (bf16): the gradients of sum(dout * o) with respect to
 * q, k and v, with o = softmax(scale * q k^T) v under the same causal /
 * window / GQA rules.  The pages name training as a use of the fused method
 * (FlashAttention explainer, "Overview"; FlashAttention-3 article, "Benefits
 * of FlashAttention-3") but print no backward algorithm; this computes the
 * derivative of the forward definition:
 *   P = exp(scale q k^T - lse), dv = P^T dout, dP = dout v^T,
 *   delta = rowsum(dout * o), dS = P * (dP - delta),
 *   dq = scale dS k, dk = scale dS^T q  (dk, dv summed over a GQA group).
 * The probabilities are recomputed from the forward's lse; nothing of size
 * Sq x Sk is stored.
 *
 *   q, o, dout, dq : bf16 [B, Hq, Sq, D].   k, v, dk, dv: bf16 [B, Hkv, Sk, D].
 *   lse            : fp32 [B, Hq, Sq], as written by attn_fwd for the same
 *                    q, k, v and mask (-inf for rows with no visible key).
 *   delta          : caller-owned fp32 scratch of B*Hq*Sq floats; on return it
 *                    holds rowsum(dout * o).
 * Rows or keys that see nothing get zero gradients.  Two launches on `stream`
 * (dq and delta, then dk and dv).  Same validation and errors as attn_fwd;
 * ATTN_ERR_NULL if any pointer needed for a non-empty output is NULL.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta,
             int B, int Hq, int Hkv, int Sq, int Sk, int D,
             int causal, int window, float scale, hipStream_t stream);

/*
 * Single-token decode against a KV cache, bf16, scale = 1/sqrt(D), split-KV.
 *
 *   q, o           : bf16 [B, Hq, D].   kcache, vcache: bf16 [B, Hkv, Sk, D].
 *   num_splits     : 1 <= num_splits <= max(Sk, 1).  Chunk c covers keys
 *                    [c*L, min((c+1)*L, Sk)), L = ceil(Sk / num_splits); an
 *                    empty chunk is the merge identity.
 * Two launches on `stream`: the split kernel writes one (m, l, acc) partial
 * per (b, h, chunk); the combine kernel merges them with the log-sum-exp
 * operator along a balanced binary tree over the chunk index and writes o.
 * Uses a library-owned workspace per device that grows on demand (the first
 * call at a new size allocates, which synchronises the device).  Calls that
 * overlap in time on one device race on that workspace; use attn_decode_ex
 * with a caller workspace for concurrent streams.
 */
int attn_decode(const void* q, const void* kcache, const void* vcache, void* o,
                int B, int Hq, int Hkv, int Sk, int D, int num_splits, hipStream_t stream);

/*
 * attn_decode with an explicit scale, an optional lse output (fp32 [B, Hq],
 * NULL to skip) and a caller-owned device workspace of at least
 * attn_decode_workspace_bytes(B, Hq, D, num_splits) bytes.  Never allocates.
 * The workspace contents on entry do not matter; it is scratch only.
 */
int attn_decode_ex(const void* q, const void* kcache, const void* vcache, void* o, float* lse,
                   int B, int Hq, int Hkv, int Sk, int D, int num_splits, float scale,
                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: attn_decode_ex
 * without a workspace argument.  The partials go to a static device array of
 * ATTN_DECODE_NOALLOC_BYTES inside the library (one per GPU, held until the
 * process ends); the call itself allocates nothing.
 *
 *   Arguments and results as attn_decode_ex.  ATTN_ERR_WORKSPACE when
 *   attn_decode_workspace_bytes(B, Hq, D, num_splits) exceeds
 *   ATTN_DECODE_NOALLOC_BYTES (32 MiB: e.g. B*Hq = 512 rows at D = 128 with
 *   up to 125 splits, or one row with up to 64 K splits).
 * The array needs no clearing (every partial is written before it is read)
 * and keeps whatever the last call left in it.  All calls on one GPU share
 * it: calls that overlap in time on one GPU (two streams, two threads) race
 * and corrupt each other's partials -- serialise them, or use attn_decode_ex
 * with one workspace per stream.  The first call on a device looks up the
 * array's device address (no allocation); that lookup fails with
 * ATTN_ERR_HIP if the library's code object cannot be loaded on the device.
 */
#define ATTN_DECODE_NOALLOC_BYTES ((size_t)32 << 20)
int attn_decode_noalloc(const void* q, const void* kcache, const void* vcache, void* o, float* lse,
                        int B, int Hq, int Hkv, int Sk, int D, int num_splits, float scale,
                        hipStream_t stream);

/*
 * Workspace bytes attn_decode_ex needs: one fp32 (m, l, acc[D]) partial per
 * (b, h, chunk), B*Hq*num_splits*(D+2)*4, plus room for the upper tree levels
 * when num_splits exceeds the 256 partials one combine workgroup merges.
 * Returns 0 for invalid arguments.  Pure host function.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int D, int num_splits);

/* Static, NUL-terminated name of a status code.  Pure host function. */
const char* attn_error_string(int status);

/* Library version string, e.g. "exact-attention gfx950 0.1".  Pure host function. */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_ATTN_H */
