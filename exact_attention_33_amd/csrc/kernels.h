// Host-side launchers of the gfx950 kernels (internal to libattn.so).
// Arguments have been validated by the C-ABI layer before these are called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ea {

// A dispatch counts its work-items (grid blocks x block threads) in 32 bits;
// the host checks each launch geometry against this before any launch.
constexpr int64_t kMaxDispatchItems = 0xffffffffLL;
inline bool dispatch_fits(int64_t blocks, int64_t threads) {
  return blocks >= 0 && blocks <= kMaxDispatchItems / threads;
}

// fp32 prefill geometry: query rows and threads per workgroup.
constexpr int kF32Rows = 16;
constexpr int kF32Threads = 1024;

struct FwdShape {
  int B, Hq, Hkv, Sq, Sk, D;
  int causal, window;
  float scale;
};

// Prefill, bf16 tensors (raw 16-bit words), one launch.
hipError_t launch_fwd_bf16(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                           float* lse, const FwdShape& s, hipStream_t stream);

// Prefill on fp8 (e4m3) codes with per-tensor descales, bf16 o, D = 64 or 128; one launch.
hipError_t launch_fwd_fp8(const uint8_t* q, const uint8_t* k, const uint8_t* v, uint16_t* o, float* lse,
                          const FwdShape& s, float q_descale, float k_descale, float v_descale,
                          hipStream_t stream);

// Prefill, fp32 tensors, one launch.
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const FwdShape& s, hipStream_t stream);

// Backward: dq (and delta = rowsum(dout * o)), then dk and dv; two launches.
hipError_t launch_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                      const uint16_t* dout, const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                      float* delta, const FwdShape& s, hipStream_t stream);

struct DecodeShape {
  int B, Hq, Hkv, Sk, D, num_splits;
  float scale;
};

// Number of (m, l, acc[D]) partial slots per (b, h) the decode needs: the
// split level plus every upper level of the combine tree.
int64_t decode_partial_slots(int num_splits);

// Split-KV decode: split kernel, then one combine pass per tree level above
// 256 partials.  `ws` holds decode_partial_slots(ns) * B*Hq*(D+2) floats.
hipError_t launch_decode(const uint16_t* q, const uint16_t* k, const uint16_t* v, uint16_t* o,
                         float* lse, const DecodeShape& s, float* ws, hipStream_t stream);

}  // namespace ea
