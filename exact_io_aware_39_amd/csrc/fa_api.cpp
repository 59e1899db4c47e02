// fa_api.cpp - the C ABI of libfa.so: argument validation and dispatch.
//
// Every check runs on the host before any HIP call, so a rejected call has no
// side effect on the device and the checks can be exercised without a GPU.
// There is no fallback path: an unsupported head size is an error, never a
// silent switch to a slower kernel.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <climits>

#include "../../include/fa.h"
#include "fa_launch.hpp"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape, scale and mask checks shared by every entry point.  `wide`: the
// entry point also has kernels for d = 256 (the bf16 forward and backward);
// the others take d = 64 and 128 only.
fa_status check_common(int B, int H, int N, int d, float scale, int causal, bool wide = false) {
  if (B <= 0 || H <= 0 || N <= 0) return FA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128 && !(wide && d == 256)) return FA_ERR_UNSUPPORTED;
  if (scale < 0.f) return FA_ERR_UNSUPPORTED;
  if (N > (1 << 20)) return FA_ERR_UNSUPPORTED;
  const int64_t bh = (int64_t)B * H;
  if (bh > (1 << 20)) return FA_ERR_UNSUPPORTED;
  if (bh * N * d >= ((int64_t)1 << 40)) return FA_ERR_UNSUPPORTED;
  // K/V tiles are staged through buffer descriptors whose 32-bit offsets span
  // 64 rows of the [B, N, H, d] tensors.
  if ((int64_t)H * d > (1 << 24)) return FA_ERR_UNSUPPORTED;
  // The largest grid any kernel uses: one workgroup per 64 rows of each head.
  if (bh * ((N + 63) / 64) > INT_MAX) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa_status check_tensors(std::initializer_list<const void*> tensors, std::initializer_list<const void*> stats) {
  for (const void* p : tensors)
    if (p == nullptr || !aligned(p, 16)) return FA_ERR_INVALID_ARG;
  for (const void* p : stats)
    if (p == nullptr || !aligned(p, 4)) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

fa_status to_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

// Decode checks: the shared limits with N = Nk, then the query rows and chunks.
fa_status check_decode(int B, int H, int Nq, int Nk, int d, float scale, int causal, int splits) {
  fa_status st = check_common(B, H, Nk, d, scale, causal);
  if (st != FA_OK) return st;
  if (Nq <= 0 || splits < 0) return FA_ERR_INVALID_ARG;
  if (causal && Nq > Nk) return FA_ERR_INVALID_ARG;
  if (Nq > 32 || splits > fa::kDecodeMaxSplits) return FA_ERR_UNSUPPORTED;
  const int64_t S = splits ? splits : fa::decode_splits(B, H, Nq, Nk);
  if ((int64_t)B * H * S > INT_MAX) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

// 16-bit keep threshold t = round(p 2^16) (ties to even, at most 2^16 - 1)
// of a dropout rate in [0, 1), and the scale 2^16 / (2^16 - t) of kept
// probabilities (the inverse of the keep probability 1 - t 2^-16).
fa::DropParams drop_params(float p, uint64_t seed, uint32_t offset) {
  fa::DropParams dp;
  dp.key0 = (uint32_t)(seed & 0xFFFFFFFFu);
  dp.key1 = (uint32_t)(seed >> 32);
  dp.offset = offset;
  const double r = std::nearbyint((double)p * 65536.0);   // default rounding: to nearest, ties to even
  const uint32_t t = r >= 65535.0 ? 65535u : (uint32_t)r;
  dp.thr = t << 16;
  dp.inv_keep = (float)(65536.0 / (double)(65536u - t));
  return dp;
}

}  // namespace

extern "C" {

fa_status fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int B, int H, int N, int d, float scale, int causal, void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal, true);
  if (st == FA_OK) st = check_tensors({Q, K, V, O}, {LSE});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  return to_status(fa::launch_fwd_bf16(Q, K, V, O, LSE, s, static_cast<hipStream_t>(stream)));
}

fa_status fa_forward_cross(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           int B, int H, int Nq, int Nk, int d, float scale, int causal,
                           void* stream) {
  fa_status st = check_common(B, H, Nq, d, scale, causal, true);
  if (st == FA_OK) st = check_common(B, H, Nk, d, scale, causal, true);
  if (st == FA_OK && causal && Nq > Nk) st = FA_ERR_INVALID_ARG;
  if (st == FA_OK) st = check_tensors({Q, K, V, O}, {LSE});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, Nq, d, scale, causal};
  return to_status(fa::launch_fwd_cross_bf16(Q, K, V, O, LSE, s, Nk, static_cast<hipStream_t>(stream)));
}

fa_status fa_forward_dropout(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             int B, int H, int N, int d, float scale, int causal, float p_drop,
                             uint64_t seed, uint32_t offset, void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal, true);
  if (st == FA_OK && !(p_drop >= 0.f && p_drop < 1.f)) st = FA_ERR_INVALID_ARG;
  if (st == FA_OK) st = check_tensors({Q, K, V, O}, {LSE});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  const fa::DropParams dp = drop_params(p_drop, seed, offset);
  // t = 0 keeps every element with multiplier 1: the plain forward computes that.
  if (dp.thr == 0) return to_status(fa::launch_fwd_bf16(Q, K, V, O, LSE, s, static_cast<hipStream_t>(stream)));
  return to_status(fa::launch_fwd_dropout_bf16(Q, K, V, O, LSE, s, dp, static_cast<hipStream_t>(stream)));
}

fa_status fa_backward_dropout(const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                              float* workspace, int B, int H, int N, int d, float scale, int causal,
                              float p_drop, uint64_t seed, uint32_t offset, void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal, true);
  if (st == FA_OK && !(p_drop >= 0.f && p_drop < 1.f)) st = FA_ERR_INVALID_ARG;
  if (st == FA_OK) st = check_tensors({Q, K, V, O, dO, dQ, dK, dV}, {LSE, workspace});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  const fa::DropParams dp = drop_params(p_drop, seed, offset);
  // t = 0 keeps every element with multiplier 1: the plain backward computes that.
  if (dp.thr == 0)
    return to_status(fa::launch_bwd_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, s,
                                         static_cast<hipStream_t>(stream)));
  return to_status(fa::launch_bwd_dropout_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, s, dp,
                                               static_cast<hipStream_t>(stream)));
}

fa_status fa_forward_fp8(const void* Q, const void* K, const void* V, float q_descale,
                         float k_descale, float v_descale, void* O, float* LSE, void* workspace,
                         int B, int H, int Nq, int Nk, int d, float scale, int causal,
                         void* stream) {
  fa_status st = check_common(B, H, Nq, d, scale, causal);
  if (st == FA_OK) st = check_common(B, H, Nk, d, scale, causal);
  if (st == FA_OK && causal && Nq > Nk) st = FA_ERR_INVALID_ARG;
  // A non-positive product of descales would turn the -inf of masked scores
  // into +inf or NaN.
  for (float x : {q_descale, k_descale, v_descale})
    if (st == FA_OK && !(std::isfinite(x) && x > 0.f)) st = FA_ERR_INVALID_ARG;
  if (st == FA_OK && !std::isfinite(scale * q_descale * k_descale)) st = FA_ERR_INVALID_ARG;
  if (st == FA_OK) st = check_tensors({Q, K, V, O, workspace}, {LSE});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, Nq, d, scale, causal};
  return to_status(fa::launch_fwd_fp8(Q, K, V, q_descale, k_descale, v_descale, O, LSE, workspace, s,
                                      Nk, static_cast<hipStream_t>(stream)));
}

size_t fa_forward_fp8_workspace_bytes(int B, int H, int Nk, int d) {
  if (check_common(B, H, Nk, d, 1.f, 0) != FA_OK) return 0;
  return fa::fwd_fp8_workspace_bytes(B, H, Nk, d);
}

fa_status fa_forward_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                         int B, int H, int N, int d, float scale, int causal, void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal);
  if (st == FA_OK) st = check_tensors({Q, K, V, O}, {LSE});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  return to_status(fa::launch_fwd_f32(Q, K, V, O, LSE, s, static_cast<hipStream_t>(stream)));
}

fa_status fa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* LSE, void* dQ, void* dK, void* dV, float* workspace,
                      int B, int H, int N, int d, float scale, int causal, void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal, true);
  if (st == FA_OK) st = check_tensors({Q, K, V, O, dO, dQ, dK, dV}, {LSE, workspace});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  return to_status(fa::launch_bwd_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, s,
                                       static_cast<hipStream_t>(stream)));
}

fa_status fa_backward_cross(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                            const float* LSE, void* dQ, void* dK, void* dV, float* workspace,
                            int B, int H, int Nq, int Nk, int d, float scale, int causal, void* stream) {
  fa_status st = check_common(B, H, Nq, d, scale, causal, true);
  if (st == FA_OK) st = check_common(B, H, Nk, d, scale, causal, true);
  if (st == FA_OK && causal && Nq > Nk) st = FA_ERR_INVALID_ARG;
  if (st == FA_OK) st = check_tensors({Q, K, V, O, dO, dQ, dK, dV}, {LSE, workspace});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, Nq, d, scale, causal};
  return to_status(fa::launch_bwd_cross_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, s, Nk,
                                             static_cast<hipStream_t>(stream)));
}

fa_status fa_backward_preprocess(const void* O, const void* dO, const float* LSE, float* workspace,
                                 int B, int H, int N, int d, void* stream) {
  fa_status st = check_common(B, H, N, d, 1.f, 0, true);
  if (st == FA_OK) st = check_tensors({O, dO}, {LSE, workspace});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, 1.f, 0};
  return to_status(fa::launch_bwd_pre_bf16(O, dO, LSE, workspace, s, static_cast<hipStream_t>(stream)));
}

fa_status fa_backward_dqdkdv(const void* Q, const void* K, const void* V, const void* dO,
                             const float* workspace, void* dQ, void* dK, void* dV,
                             int B, int H, int N, int d, float scale, int causal, void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal, true);
  if (st == FA_OK) st = check_tensors({Q, K, V, dO, dQ, dK, dV}, {workspace});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  return to_status(fa::launch_bwd_dqdkdv_bf16(Q, K, V, dO, workspace, dQ, dK, dV, s,
                                              static_cast<hipStream_t>(stream)));
}

fa_status fa_backward_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                           const float* workspace, void* dK, void* dV,
                           int B, int H, int N, int d, float scale, int causal, void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal, true);
  if (st == FA_OK) st = check_tensors({Q, K, V, dO, dK, dV}, {workspace});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  return to_status(fa::launch_bwd_dkdv_bf16(Q, K, V, dO, workspace, dK, dV, s,
                                            static_cast<hipStream_t>(stream)));
}

fa_status fa_backward_dq(const void* Q, const void* K, const void* V, const void* dO,
                         const float* workspace, void* dQ,
                         int B, int H, int N, int d, float scale, int causal, void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal, true);
  if (st == FA_OK) st = check_tensors({Q, K, V, dO, dQ}, {workspace});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  return to_status(fa::launch_bwd_dq_bf16(Q, K, V, dO, workspace, dQ, s,
                                          static_cast<hipStream_t>(stream)));
}

fa_status fa_backward_f32(const float* Q, const float* K, const float* V, const float* O,
                          const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                          float* workspace, int B, int H, int N, int d, float scale, int causal,
                          void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal);
  if (st == FA_OK) st = check_tensors({Q, K, V, O, dO, dQ, dK, dV}, {LSE, workspace});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  return to_status(fa::launch_bwd_f32(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, s,
                                      static_cast<hipStream_t>(stream)));
}

fa_status fa_decode(const void* Q, const void* K, const void* V, void* O, float* LSE,
                    float* workspace, int B, int H, int Nq, int Nk, int d, float scale,
                    int causal, int splits, void* stream) {
  fa_status st = check_decode(B, H, Nq, Nk, d, scale, causal, splits);
  if (st == FA_OK) st = check_tensors({Q, K, V, O}, {LSE, workspace});
  if (st != FA_OK) return st;
  const int S = splits ? splits : fa::decode_splits(B, H, Nq, Nk);
  const fa::DecodeShape s{B, H, Nq, Nk, d, scale, causal, S};
  return to_status(fa::launch_decode_bf16(Q, K, V, O, LSE, workspace, s,
                                          static_cast<hipStream_t>(stream)));
}

int fa_decode_splits(int B, int H, int Nq, int Nk, int d) {
  if (check_decode(B, H, Nq, Nk, d, 1.f, 0, 0) != FA_OK) return 0;
  return fa::decode_splits(B, H, Nq, Nk);
}

size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d, int splits) {
  if (check_decode(B, H, Nq, Nk, d, 1.f, 0, splits) != FA_OK) return 0;
  const size_t S = splits ? (size_t)splits : (size_t)fa::decode_splits(B, H, Nq, Nk);
  return (size_t)B * H * S * Nq * (d + 1) * sizeof(float);
}

fa_status fa_backward_single_pass(const void* Q, const void* K, const void* V, const void* O,
                                  const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                  float* workspace, int B, int H, int N, int d, float scale, int causal,
                                  void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal);
  if (st == FA_OK) st = check_tensors({Q, K, V, O, dO, dQ, dK, dV, workspace}, {LSE});
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  return to_status(fa::launch_bwd_single_pass_bf16(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, s,
                                                   static_cast<hipStream_t>(stream)));
}

size_t fa_backward_single_pass_workspace_bytes(int B, int H, int N, int d) {
  if (check_common(B, H, N, d, 1.f, 0) != FA_OK) return 0;
  return ((size_t)fa::bwd_single_pass_acc_offset(B, H, N) + (size_t)B * N * H * d) * sizeof(float);
}

fa_status fa_backward_noalloc(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                              const float* LSE, void* dQ, void* dK, void* dV,
                              int B, int H, int N, int d, float scale, int causal, void* stream) {
  fa_status st = check_common(B, H, N, d, scale, causal, true);
  if (st == FA_OK) st = check_tensors({Q, K, V, O, dO, dQ, dK, dV}, {LSE});
  if (st == FA_OK && (int64_t)B * H * N > fa::kNoallocMaxRows) st = FA_ERR_SCRATCH_LIMIT;
  if (st != FA_OK) return st;
  const fa::AttnShape s{B, H, N, d, scale, causal};
  return to_status(fa::launch_bwd_bf16_noalloc(Q, K, V, O, dO, LSE, dQ, dK, dV, s,
                                               static_cast<hipStream_t>(stream)));
}

size_t fa_backward_workspace_bytes(int B, int H, int N, int d) {
  if (check_common(B, H, N, d, 1.f, 0, true) != FA_OK) return 0;
  return 2 * (size_t)B * H * N * sizeof(float);
}

const char* fa_status_string(fa_status status) {
  switch (status) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARG: return "FA_ERR_INVALID_ARG: invalid argument (null or misaligned pointer, bad size, scale or mask flag)";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: unsupported configuration (head size without kernels for this entry point, negative scale, or size limits)";
    case FA_ERR_LAUNCH: return "FA_ERR_LAUNCH: a HIP launch failed";
    case FA_ERR_SCRATCH_LIMIT: return "FA_ERR_SCRATCH_LIMIT: fa_backward_noalloc needs B*H*N <= 2^21 query rows (its static scratch holds 16 MiB); use fa_backward with a workspace";
    default: return "unknown fa_status";
  }
}

}  // extern "C"
