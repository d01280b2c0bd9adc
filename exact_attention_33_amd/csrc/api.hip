// C-ABI entry points of libattn.so (declared in include/attn.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so an invalid call enqueues nothing and writes nothing.  No
// C++ exception crosses this boundary.
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/attn.h"
#include "kernels.h"

namespace {

constexpr int kMaxSeq = 1 << 29;  // keeps positions +- window inside int32 in the kernels

int check_common(int B, int Hq, int Hkv, int Sq, int Sk, int D) {
  if (B < 0 || Hq < 0 || Hkv < 0 || Sq < 0 || Sk < 0) return ATTN_ERR_SHAPE;
  if (Sq > kMaxSeq || Sk > kMaxSeq) return ATTN_ERR_SHAPE;
  if (Hq > 0 && (Hkv < 1 || Hq % Hkv != 0)) return ATTN_ERR_GQA;
  if (D != 64 && D != 128) return ATTN_ERR_HEADDIM;
  return ATTN_OK;
}

// The kernels move q, k, v, o (and the gradients) in 16-byte vectors and
// lse, delta and the decode workspace in 4- and 16-byte words.
bool misaligned(const void* p, uintptr_t bytes) {
  return p != nullptr && ((uintptr_t)p % bytes) != 0;
}

int check_scale(float scale) {
  return (isfinite(scale) && scale > 0.f) ? ATTN_OK : ATTN_ERR_ARG;
}

// Prefill argument check (shared by the bf16 and fp32 entry points).
int check_fwd(const void* q, const void* k, const void* v, const void* o, int B, int Hq, int Hkv,
              int Sq, int Sk, int D, int causal, int window, float scale) {
  int st = check_common(B, Hq, Hkv, Sq, Sk, D);
  if (st != ATTN_OK) return st;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  if (window < -1) return ATTN_ERR_WINDOW;
  if ((st = check_scale(scale)) != ATTN_OK) return st;
  const int64_t rows = (int64_t)B * Hq * Sq;
  if (rows == 0) return ATTN_OK;  // nothing to read or write
  if (q == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (Sk > 0 && (k == nullptr || v == nullptr)) return ATTN_ERR_NULL;
  if (misaligned(q, 16) || misaligned(k, 16) || misaligned(v, 16) || misaligned(o, 16))
    return ATTN_ERR_ARG;
  const int64_t bh = (int64_t)B * Hq;
  if (bh > INT32_MAX / 8) return ATTN_ERR_SHAPE;
  // bf16 / fp8 prefill (and the backward's dq pass): 256-row workgroups of
  // 512 threads, or 128-row ones of 256
  if (!ea::dispatch_fits(((int64_t)Sq + 255) / 256 * bh, 512) ||
      !ea::dispatch_fits(((int64_t)Sq + 127) / 128 * bh, 256))
    return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

int check_decode(const void* q, const void* kc, const void* vc, const void* o, int B, int Hq,
                 int Hkv, int Sk, int D, int num_splits, float scale) {
  int st = check_common(B, Hq, Hkv, 1, Sk, D);
  if (st != ATTN_OK) return st;
  if (num_splits < 1 || num_splits > (Sk > 1 ? Sk : 1)) return ATTN_ERR_SPLITS;
  if ((st = check_scale(scale)) != ATTN_OK) return st;
  const int64_t bh = (int64_t)B * Hq;
  if (bh == 0) return ATTN_OK;
  if (q == nullptr || o == nullptr) return ATTN_ERR_NULL;
  if (Sk > 0 && (kc == nullptr || vc == nullptr)) return ATTN_ERR_NULL;
  if (misaligned(q, 16) || misaligned(kc, 16) || misaligned(vc, 16) || misaligned(o, 16))
    return ATTN_ERR_ARG;
  // split kernel: one 256-thread workgroup per (chunk, kv head, batch row,
  // group of 16 query heads); combine: one per (b, h, group of 256 partials)
  const int64_t nhg = ((Hq / Hkv) + 15) / 16;
  if (!ea::dispatch_fits((int64_t)num_splits * Hkv * B * nhg, 256)) return ATTN_ERR_SHAPE;
  if (!ea::dispatch_fits(bh * (((int64_t)num_splits + 255) / 256), 256)) return ATTN_ERR_SHAPE;
  return ATTN_OK;
}

int to_status(hipError_t e) { return e == hipSuccess ? ATTN_OK : ATTN_ERR_HIP; }

ea::FwdShape fwd_shape(int B, int Hq, int Hkv, int Sq, int Sk, int D, int causal, int window,
                       float scale) {
  ea::FwdShape s;
  s.B = B;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.Sq = Sq;
  s.Sk = Sk;
  s.D = D;
  s.causal = causal;
  // a half width that covers every (query, key) pair is no window at all
  s.window = ((int64_t)window >= (int64_t)Sq + Sk) ? -1 : window;
  s.scale = scale;
  return s;
}

// Library-owned decode workspace, one grow-only buffer per device.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws;

int library_workspace(size_t need, void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  if ((size_t)dev >= g_ws.size()) g_ws.resize(dev + 1);
  Workspace& w = g_ws[dev];
  if (w.bytes < need) {
    if (w.ptr != nullptr) {
      if (hipFree(w.ptr) != hipSuccess) return ATTN_ERR_HIP;
      w.ptr = nullptr;
      w.bytes = 0;
    }
    if (hipMalloc(&w.ptr, need) != hipSuccess) {
      w.ptr = nullptr;
      return ATTN_ERR_HIP;
    }
    w.bytes = need;
  }
  *out = w.ptr;
  return ATTN_OK;
}

// Scratch memory of attn_decode_noalloc: a static device array, one copy per
// GPU the library runs on, held until the process ends.  Host code never
// names `scratch` as an address: the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
constexpr size_t kNoAllocBytes = ATTN_DECODE_NOALLOC_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};  // per device: the address of `scratch` on it

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return ATTN_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

size_t attn_decode_workspace_bytes(int B, int Hq, int D, int num_splits) {
  if (B < 0 || Hq < 0 || num_splits < 1 || (D != 64 && D != 128)) return 0;
  return (size_t)ea::decode_partial_slots(num_splits) * (size_t)B * (size_t)Hq * (size_t)(D + 2) *
         sizeof(float);
}

const char* attn_error_string(int status) {
  switch (status) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL: return "ATTN_ERR_NULL: a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE: a size is negative or too large";
    case ATTN_ERR_GQA: return "ATTN_ERR_GQA: Hq must be a positive multiple of Hkv";
    case ATTN_ERR_HEADDIM: return "ATTN_ERR_HEADDIM: D must be 64 or 128";
    case ATTN_ERR_SPLITS: return "ATTN_ERR_SPLITS: need 1 <= num_splits <= max(Sk, 1)";
    case ATTN_ERR_WINDOW: return "ATTN_ERR_WINDOW: window must be -1 or a half width >= 0";
    case ATTN_ERR_WORKSPACE: return "ATTN_ERR_WORKSPACE: workspace missing or too small";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP: the HIP runtime reported an error";
    case ATTN_ERR_ARG:
      return "ATTN_ERR_ARG: causal must be 0/1, scale finite and > 0, tensors 16-byte and lse 4-byte aligned";
    default: return "unknown attn status";
  }
}

const char* attn_version(void) { return "exact-attention gfx950 0.1"; }

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Sq, int Sk, int D, int causal, int window, float scale,
             hipStream_t stream) {
  int st = check_fwd(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, window, scale);
  if (st != ATTN_OK || (int64_t)B * Hq * Sq == 0) return st;
  if (misaligned(lse, 4)) return ATTN_ERR_ARG;
  return to_status(ea::launch_fwd_bf16((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                       (uint16_t*)o, lse,
                                       fwd_shape(B, Hq, Hkv, Sq, Sk, D, causal, window, scale),
                                       stream));
}

int attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
                 int Hq, int Hkv, int Sq, int Sk, int D, int causal, int window, float scale,
                 hipStream_t stream) {
  int st = check_fwd(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, window, scale);
  if (st != ATTN_OK || (int64_t)B * Hq * Sq == 0) return st;
  if (misaligned(lse, 4)) return ATTN_ERR_ARG;
  if (!ea::dispatch_fits(((int64_t)Sq + ea::kF32Rows - 1) / ea::kF32Rows * B * Hq, ea::kF32Threads))
    return ATTN_ERR_SHAPE;
  return to_status(ea::launch_fwd_f32(q, k, v, o, lse,
                                      fwd_shape(B, Hq, Hkv, Sq, Sk, D, causal, window, scale),
                                      stream));
}

int attn_fwd_fp8(const void* q8, const void* k8, const void* v8, void* o, float* lse, int B, int Hq,
                 int Hkv, int Sq, int Sk, int D, int causal, int window, float scale,
                 float q_descale, float k_descale, float v_descale, hipStream_t stream) {
  int st = check_fwd(q8, k8, v8, o, B, Hq, Hkv, Sq, Sk, D, causal, window, scale);
  if (st != ATTN_OK) return st;
  if (check_scale(q_descale) != ATTN_OK || check_scale(k_descale) != ATTN_OK ||
      check_scale(v_descale) != ATTN_OK)
    return ATTN_ERR_ARG;
  if ((int64_t)B * Hq * Sq == 0) return ATTN_OK;
  if (misaligned(lse, 4)) return ATTN_ERR_ARG;
  return to_status(ea::launch_fwd_fp8((const uint8_t*)q8, (const uint8_t*)k8, (const uint8_t*)v8,
                                      (uint16_t*)o, lse,
                                      fwd_shape(B, Hq, Hkv, Sq, Sk, D, causal, window, scale),
                                      q_descale, k_descale, v_descale, stream));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int Hq, int Hkv,
             int Sq, int Sk, int D, int causal, int window, float scale, hipStream_t stream) {
  int st = check_fwd(q, k, v, o, B, Hq, Hkv, Sq, Sk, D, causal, window, scale);
  if (st != ATTN_OK) return st;
  const int64_t rows = (int64_t)B * Hq * Sq, keys = (int64_t)B * Hkv * Sk;
  if (rows == 0 && keys == 0) return ATTN_OK;
  if (rows > 0 && (q == nullptr || o == nullptr || dout == nullptr || lse == nullptr ||
                   dq == nullptr || delta == nullptr))
    return ATTN_ERR_NULL;
  if (keys > 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr))
    return ATTN_ERR_NULL;
  if (misaligned(dout, 16) || misaligned(dq, 16) || misaligned(dk, 16) || misaligned(dv, 16) ||
      misaligned(lse, 4) || misaligned(delta, 4))
    return ATTN_ERR_ARG;
  // dk/dv pass: 128-key workgroups of 256 threads
  if (!ea::dispatch_fits(((int64_t)Sk + 127) / 128 * B * Hkv, 256)) return ATTN_ERR_SHAPE;
  return to_status(ea::launch_bwd((const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                                  (const uint16_t*)o, (const uint16_t*)dout, lse, (uint16_t*)dq,
                                  (uint16_t*)dk, (uint16_t*)dv, delta,
                                  fwd_shape(B, Hq, Hkv, Sq, Sk, D, causal, window, scale), stream));
}

int attn_decode_ex(const void* q, const void* kcache, const void* vcache, void* o, float* lse,
                   int B, int Hq, int Hkv, int Sk, int D, int num_splits, float scale,
                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_decode(q, kcache, vcache, o, B, Hq, Hkv, Sk, D, num_splits, scale);
  if (st != ATTN_OK || (int64_t)B * Hq == 0) return st;
  if (workspace == nullptr || workspace_bytes < attn_decode_workspace_bytes(B, Hq, D, num_splits))
    return ATTN_ERR_WORKSPACE;
  if (misaligned(lse, 4) || misaligned(workspace, 16)) return ATTN_ERR_ARG;
  ea::DecodeShape s;
  s.B = B;
  s.Hq = Hq;
  s.Hkv = Hkv;
  s.Sk = Sk;
  s.D = D;
  s.num_splits = num_splits;
  s.scale = scale;
  return to_status(ea::launch_decode((const uint16_t*)q, (const uint16_t*)kcache,
                                     (const uint16_t*)vcache, (uint16_t*)o, lse, s,
                                     (float*)workspace, stream));
}

int attn_decode_noalloc(const void* q, const void* kcache, const void* vcache, void* o, float* lse,
                        int B, int Hq, int Hkv, int Sk, int D, int num_splits, float scale,
                        hipStream_t stream) {
  int st = check_decode(q, kcache, vcache, o, B, Hq, Hkv, Sk, D, num_splits, scale);
  if (st != ATTN_OK || (int64_t)B * Hq == 0) return st;
  const size_t need = attn_decode_workspace_bytes(B, Hq, D, num_splits);
  if (need > kNoAllocBytes) return ATTN_ERR_WORKSPACE;
  if (misaligned(lse, 4)) return ATTN_ERR_ARG;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != ATTN_OK) return st;
  return attn_decode_ex(q, kcache, vcache, o, lse, B, Hq, Hkv, Sk, D, num_splits, scale, ws, need,
                        stream);
}

int attn_decode(const void* q, const void* kcache, const void* vcache, void* o, int B, int Hq,
                int Hkv, int Sk, int D, int num_splits, hipStream_t stream) {
  const float scale = 1.0f / sqrtf((float)D);
  int st = check_decode(q, kcache, vcache, o, B, Hq, Hkv, Sk, D, num_splits, scale);
  if (st != ATTN_OK || (int64_t)B * Hq == 0) return st;
  const size_t need = attn_decode_workspace_bytes(B, Hq, D, num_splits);
  void* ws = nullptr;
  if ((st = library_workspace(need, &ws)) != ATTN_OK) return st;
  return attn_decode_ex(q, kcache, vcache, o, nullptr, B, Hq, Hkv, Sk, D, num_splits, scale, ws,
                        need, stream);
}

}  // extern "C"
