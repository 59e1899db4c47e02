// fa_launch.hpp - host-side launchers shared by the C ABI and the kernel files.
// Every launcher assumes arguments already validated by fa_api.cpp and returns
// the hipError_t of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct AttnShape {
  int B, H, N, d;
  float scale;
  int causal;
};

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                           const AttnShape& s, hipStream_t stream);
// Forward with N query rows against Nk key rows; with a causal mask query row
// i is sequence position Nk - N + i.
hipError_t launch_fwd_cross_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                 const AttnShape& s, int Nk, hipStream_t stream);
// FP8 forward (e4m3 Q, K, V with descales); `ws` holds V^T, fwd_fp8_workspace_bytes.
size_t fwd_fp8_workspace_bytes(int B, int H, int Nk, int d);
hipError_t launch_fwd_fp8(const void* q, const void* k, const void* v, float dq, float dk, float dv,
                          void* o, float* lse, void* ws, const AttnShape& s, int Nk, hipStream_t stream);
// Dropout on the probabilities: element (query row i, key j) of head bh is
// kept when 16-bit field 4 ((j >> 3) & 1) + (j & 3) (field f: the low half of
// word f / 2 for even f, the high half for odd f) of Philox4x32-10 on the
// counter (2 (j >> 4) + ((j >> 2) & 1), i, bh, offset) under the key
// (key0, key1) is >= t = round(p 2^16); kept probabilities are scaled by
// inv_keep = 2^16 / (2^16 - t).
struct DropParams {
  uint32_t key0, key1;   // seed, low and high word
  uint32_t offset;       // fourth counter word (one mask per offset)
  uint32_t thr;          // t << 16 (a field f is kept when f << 16 >= thr)
  float inv_keep;        // 2^16 / (2^16 - t)
};
// Forward with dropout (square attention).
hipError_t launch_fwd_dropout_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                                   const AttnShape& s, const DropParams& drop, hipStream_t stream);
// Backward of launch_fwd_dropout_bf16 (same mask), preprocess and the fused passes.
hipError_t launch_bwd_dropout_bf16(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                   float* ws, const AttnShape& s, const DropParams& drop,
                                   hipStream_t stream);
hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          const AttnShape& s, hipStream_t stream);
hipError_t launch_bwd_bf16(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv,
                           float* dvec, const AttnShape& s, hipStream_t stream);
// Backward with N query rows against Nk key rows (causal: query row i is
// sequence position Nk - N + i); Nk == N is launch_bwd_bf16.
hipError_t launch_bwd_cross_bf16(const void* q, const void* k, const void* v, const void* o,
                                 const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                 float* ws, const AttnShape& s, int Nk, hipStream_t stream);
hipError_t launch_bwd_pre_bf16(const void* o, const void* dout, const float* lse, float* ws,
                               const AttnShape& s, hipStream_t stream);
// Single-pass backward (d = 64, 128): dQ accumulated in fp32 with atomics by
// the dK/dV pass.  Workspace: [-D | -LSE log2 e | pad to 16 B | dQ acc
// (B N H d floats)], the accumulator at bwd_single_pass_acc_offset floats.
int64_t bwd_single_pass_acc_offset(int B, int H, int N);
hipError_t launch_bwd_single_pass_bf16(const void* q, const void* k, const void* v, const void* o,
                                       const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                       float* ws, const AttnShape& s, hipStream_t stream);
hipError_t launch_bwd_dkdv_bf16(const void* q, const void* k, const void* v, const void* dout,
                                const float* ws, void* dk, void* dv, const AttnShape& s,
                                hipStream_t stream);
hipError_t launch_bwd_dqdkdv_bf16(const void* q, const void* k, const void* v, const void* dout,
                                  const float* ws, void* dq, void* dk, void* dv, const AttnShape& s,
                                  hipStream_t stream);
hipError_t launch_bwd_dq_bf16(const void* q, const void* k, const void* v, const void* dout,
                              const float* ws, void* dq, const AttnShape& s, hipStream_t stream);
// Decode: Nq query rows per head against Nk keys, `splits` key chunks.
constexpr int kDecodeMaxSplits = 4096;
struct DecodeShape {
  int B, H, Nq, Nk, d;
  float scale;
  int causal;
  int splits;
};
// Number of key chunks chosen when the caller passes splits = 0.
int decode_splits(int B, int H, int Nq, int Nk);
hipError_t launch_decode_bf16(const void* q, const void* k, const void* v, void* o, float* lse,
                              float* ws, const DecodeShape& s, hipStream_t stream);

// fa_backward with its workspace in the library's static scratch array
// (fa_noalloc.hip); B H N <= kNoallocMaxRows, checked by the caller.
constexpr int64_t kNoallocMaxRows = int64_t(1) << 21;
hipError_t launch_bwd_bf16_noalloc(const void* q, const void* k, const void* v, const void* o,
                                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                                   const AttnShape& s, hipStream_t stream);

hipError_t launch_bwd_f32(const float* q, const float* k, const float* v, const float* o,
                          const float* dout, const float* lse, float* dq, float* dk, float* dv,
                          float* dvec, const AttnShape& s, hipStream_t stream);

}  // namespace fa
