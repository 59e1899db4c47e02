/*
 * fa.h - C ABI of libfa.so: fused, IO-aware exact attention for MI355X (gfx950).
 *
 * Computes O = softmax(scale * Q K^T [+ causal mask]) V for every (batch, head)
 * without writing the N x N score or probability matrices to memory, and the
 * gradients of a loss with respect to Q, K and V by recomputing the
 * probabilities from a per-row logsumexp saved by the forward.
 *
 * Sources (web pages, with the part each entry point follows):
 *   page "FlashAttention" (vagrantpi.github.io PKM note): the IO view of
 *     standard attention (S = QK^T/sqrt(d), P = softmax(S), O = PV) and its
 *     three techniques: tiling, the online-softmax recurrence (running max,
 *     running sum, rescaled unnormalised output, one final divide) and
 *     recomputation in the backward from saved row statistics.
 *   page "知识点13 | FlashAttention深度攻略" (blog.xiaohack.org): section 2
 *     (softmax(QK^T/sqrt(d_k))V), section 3 (blocks of B_r query rows and B_c
 *     key rows), section 6 (backward with recomputation), section 7 (one fused
 *     kernel), and the PyTorch module under "代码手撕环节" whose forward takes
 *     (batch, seq_len, num_heads, head_dim) tensors, uses scale = head_dim^-0.5
 *     and an optional causal mask that hides key j from query i when j > i.
 *   page "Flash Attention 到底做了什么？" (guanweilu.cn): section on the backward
 *     (keep per-row statistics, recompute S instead of storing it).
 *
 * Conventions shared by every entry point:
 *   Layout    Q, K, V, O, dO, dQ, dK, dV are dense row-major [B, N, H, d]
 *             tensors (element (b, n, h, c) at ((b*N + n)*H + h)*d + c).
 *             LSE and the backward workspace are dense float32 [B, H, N].
 *   Masking   causal = 1 hides key j from query i when j > i (absolute index,
 *             square attention: queries and keys share the length N).
 *   Scale     the float32 factor applied to Q K^T; it must be finite and >= 0
 *             (the pages use head_dim^-0.5).
 *   LSE       natural-log logsumexp of each row of scale * Q K^T (masked
 *             entries excluded): O = exp(scale q_i K^T - LSE_i) V.
 *   Ownership the caller allocates and owns every buffer (device memory of
 *             the current device).  The library allocates, frees and
 *             synchronises nothing.
 *   Streams   work is enqueued asynchronously on `stream` (a hipStream_t;
 *             NULL means the null stream).  Device faults surface at the
 *             caller's next synchronisation, as for any HIP launch.
 *   Errors    arguments are validated on the host before any HIP call:
 *               FA_ERR_INVALID_ARG  null pointer, a tensor pointer not 16-byte
 *                                   aligned, an LSE/workspace pointer not
 *                                   4-byte aligned, B, H or N <= 0, a
 *                                   non-finite scale, causal not 0 or 1;
 *               FA_ERR_UNSUPPORTED  a head size d without kernels (64, 128
 *                                   and 256 for the bf16 forward and
 *                                   backward entry points, including the
 *                                   cross-length ones and the separate
 *                                   backward passes; 64 and 128 for the
 *                                   fp32, FP8 and decode ones), scale < 0,
 *                                   or sizes beyond the limits below; there
 *                                   is no fallback path;
 *               FA_ERR_LAUNCH       a HIP call or kernel launch failed.
 *             On error nothing has been enqueued.
 *   Limits    N <= 2^20, B*H <= 2^20, H*d <= 2^24, B*N*H*d < 2^40 elements.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_LAUNCH = 3,
  FA_ERR_SCRATCH_LIMIT = 4   /* fa_backward_noalloc only: B*H*N above its scratch */
} fa_status;

/*
 * Forward, bfloat16 tensors (fp32 accumulation).  Q, K, V are read; O
 * ([B, N, H, d] bf16, rounded to nearest even) and LSE ([B, H, N] fp32) are
 * written.  Tiling and online softmax: page "FlashAttention", techniques 1
 * and 2; the saved statistics of technique 3 are returned as LSE.
 */
fa_status fa_forward(const void* Q, const void* K, const void* V, void* O, float* LSE,
                     int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * Forward with Nq query rows against Nk key rows per head, bfloat16 tensors:
 * Q and O are [B, Nq, H, d], K and V [B, Nk, H, d], LSE [B, H, Nq].
 * causal = 0: every query row sees all Nk keys (cross-attention).
 * causal = 1: query row i is sequence position Nk - Nq + i and sees keys
 * 0 .. Nk - Nq + i (rows appended after a cached prefix; requires Nq <= Nk;
 * Nq = Nk is fa_forward).  Same kernels, layouts, checks and limits as
 * fa_forward, applied to both lengths.
 */
fa_status fa_forward_cross(const void* Q, const void* K, const void* V, void* O, float* LSE,
                           int B, int H, int Nq, int Nk, int d, float scale, int causal,
                           void* stream);

/*
 * Forward with dropout on the probabilities, bfloat16 tensors (page "知识点13 |
 * FlashAttention深度攻略", section 7: the softmax step fused into the one
 * kernel carries the mask and dropout).  O = (P * Z) V with P the softmax of
 * scale Q K^T [+ causal mask] and Z_ij = keep_ij * 2^16 / (2^16 - t),
 * t = round(p_drop 2^16) (ties to even, at most 2^16 - 1: the drop rate is
 * p_drop to the nearest multiple of 2^-16, and the scale is the inverse of
 * the keep probability); LSE is that of P (unchanged by dropout).  The mask
 * is never stored: each call of Philox4x32-10 (Salmon et al., SC 2011) under
 * the key (seed mod 2^32, seed / 2^32) yields eight 16-bit fields (field f:
 * the low half of word f / 2 for even f, the high half for odd f); element
 * (query row i, key j) of head b*H + h is kept when field
 * 4 ((j / 8) % 2) + j % 4 of the call on the counter
 * (2 (j / 16) + (j / 4) % 2, i, b*H + h, offset) is >= t.
 * 0 <= p_drop < 1 (else FA_ERR_INVALID_ARG); p_drop = 0 keeps everything: a
 * rate that rounds to t = 0 runs exactly what fa_forward (and, for the
 * backward, fa_backward) runs.
 * Same layouts, checks and limits as fa_forward (square attention).
 */
fa_status fa_forward_dropout(const void* Q, const void* K, const void* V, void* O, float* LSE,
                             int B, int H, int N, int d, float scale, int causal, float p_drop,
                             uint64_t seed, uint32_t offset, void* stream);

/*
 * Backward of fa_forward_dropout with the same (p_drop, seed, offset): the
 * chain rule with the mask replayed, dV = (P * Z)^T dO, dP = (dO V^T) * Z,
 * D = rowsum(dO * O), dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 * O and LSE are the forward's; same workspace and checks as fa_backward.
 */
fa_status fa_backward_dropout(const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                              float* workspace, int B, int H, int N, int d, float scale, int causal,
                              float p_drop, uint64_t seed, uint32_t offset, void* stream);

/*
 * Forward on FP8 inputs (page "FlashAttention", part "效果": FlashAttention-3
 * and its FP8 mode; page "知识点13 | FlashAttention深度攻略", part
 * "前沿研究方向": mixed precision with FP8).  Q is [B, Nq, H, d], K and V are
 * [B, Nk, H, d], each element one byte: an OCP E4M3 code (bias 7, largest
 * magnitude 448, S.1111.111 = NaN, which propagates).  The value of an
 * element is its code's value times the tensor's descale (q_descale,
 * k_descale, v_descale: finite and > 0, else FA_ERR_INVALID_ARG).  Writes O
 * (bf16, [B, Nq, H, d]) and LSE (fp32, [B, H, Nq]) of
 *   O = softmax(scale * q_descale * k_descale * Q K^T [+ mask]) V * v_descale.
 * Both products run on FP8 matrix units with fp32 accumulation: the
 * probabilities enter the second one as E4M3 codes of 2^8 p, p taken against
 * the exact running row maximum (rounded to nearest, ties to even); the row
 * sum and LSE use the unrounded p.  The per-element error this adds to O is at
 * most v_descale * sum_j max(2^-4 2^8 p_ij, 2^-10) |V_j| / (2^8 l_i).
 * Masking as in fa_forward_cross (causal = 1: query row i is sequence
 * position Nk - Nq + i; requires Nq <= Nk).  `workspace` is caller-owned
 * device memory of fa_forward_fp8_workspace_bytes(B, H, Nk, d) bytes (a
 * transposed copy of V, [B H, d, Nk rounded up to 64], rewritten by every
 * call).  Pointers: Q, K, V, O, workspace 16-byte aligned, LSE 4-byte.  Same
 * shape limits as fa_forward_cross.
 */
fa_status fa_forward_fp8(const void* Q, const void* K, const void* V, float q_descale,
                         float k_descale, float v_descale, void* O, float* LSE, void* workspace,
                         int B, int H, int Nq, int Nk, int d, float scale, int causal,
                         void* stream);

/* Bytes of workspace fa_forward_fp8 needs: B H d (Nk rounded up to 64) (0 for invalid sizes). */
size_t fa_forward_fp8_workspace_bytes(int B, int H, int Nk, int d);

/*
 * Forward, float32 tensors: same contract as fa_forward with every tensor
 * float32 (fp32 products and accumulation throughout).
 */
fa_status fa_forward_f32(const float* Q, const float* K, const float* V, float* O, float* LSE,
                         int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * Backward, bfloat16 tensors.  Given the forward's inputs, its O and LSE
 * (unchanged), and dO = dLoss/dO, writes dQ, dK, dV (bf16, [B, N, H, d]).
 * P is rebuilt from LSE (page "FlashAttention", technique 3; page "知识点13 |
 * FlashAttention深度攻略", section 6) and the gradients follow the chain rule
 * of softmax: dV = P^T dO, dP = dO V^T, D_i = rowsum(dO * O)_i,
 * dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 * `workspace` is caller-owned device memory of fa_backward_workspace_bytes()
 * bytes; on return its first B*H*N floats hold -D ([B, H, N] fp32).
 */
fa_status fa_backward(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                      const float* LSE, void* dQ, void* dK, void* dV, float* workspace,
                      int B, int H, int N, int d, float scale, int causal, void* stream);

/*
 * Single-pass backward, bfloat16 tensors, d = 64 or 128: the same result as
 * fa_backward (same arguments, layouts and chain rule) computed with one pass
 * over the key tiles instead of two.  Page "FlashAttention" (the paragraph
 * after the "效果" table) and page "知识点13 | FlashAttention深度攻略"
 * (follow-up questions) credit FlashAttention-2 with a different division of
 * the work across the GPU; this entry point is such a division for the
 * backward: the dK/dV pass, which already forms dS for its keys, also adds dS K into an
 * fp32 dQ accumulator with atomic adds (the dQ pass and its recomputation of
 * S and dP are gone), and a last launch writes dQ = scale * acc as bf16.
 * The order of the atomic adds varies from run to run, so dQ is reproducible
 * only to fp32 rounding (dK and dV are bitwise those of fa_backward);
 * fa_backward stays the deterministic form.  `workspace` is caller-owned
 * device memory of fa_backward_single_pass_workspace_bytes() bytes, 16-byte
 * aligned: [-D | -LSE log2 e | padding to 16 bytes | the accumulator
 * (B*N*H*d floats)]; the call zeroes the accumulator itself.  Same errors as
 * fa_backward; d = 256 is FA_ERR_UNSUPPORTED.
 */
fa_status fa_backward_single_pass(const void* Q, const void* K, const void* V, const void* O,
                                  const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                                  float* workspace, int B, int H, int N, int d, float scale, int causal,
                                  void* stream);
/* Bytes of workspace fa_backward_single_pass needs (0 for invalid sizes). */
size_t fa_backward_single_pass_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward of fa_forward_cross, bfloat16 tensors: Q, O, dO, dQ are
 * [B, Nq, H, d], K, V, dK, dV [B, Nk, H, d], LSE [B, H, Nq] (the forward's,
 * unchanged).  Masking as in fa_forward_cross (causal = 1: query row i is
 * sequence position Nk - Nq + i; requires Nq <= Nk).  Same chain rule as
 * fa_backward; `workspace` holds fa_backward_workspace_bytes(B, H, Nq, d)
 * bytes and on return its first B*H*Nq floats hold -D.  Nq = Nk runs exactly
 * what fa_backward runs.  Same checks and limits as fa_forward_cross.
 */
fa_status fa_backward_cross(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                            const float* LSE, void* dQ, void* dK, void* dV, float* workspace,
                            int B, int H, int Nq, int Nk, int d, float scale, int causal,
                            void* stream);

/*
 * The three passes fa_backward runs, in this order, for callers that schedule
 * them themselves (bf16 tensors, same layouts and checks as fa_backward):
 *   fa_backward_preprocess  fills `workspace` with -D_i (D_i = sum_c dO_ic O_ic)
 *                           and -LSE_i log2(e) (two fp32 [B, H, N] arrays, in
 *                           that order);
 *   fa_backward_dqdkdv      dQ, dK and dV in one launch (what fa_backward runs
 *                           after the preprocess: both passes share one grid,
 *                           heaviest tiles first);
 *   fa_backward_dkdv        dK = scale dS^T Q and dV = P^T dO alone;
 *   fa_backward_dq          dQ = scale dS K alone;
 * the last three read the workspace written by the preprocess.  They only
 * read shared inputs, so once the preprocess has completed the separate dK/dV
 * and dQ passes may also run concurrently on different streams.
 */
fa_status fa_backward_preprocess(const void* O, const void* dO, const float* LSE, float* workspace,
                                 int B, int H, int N, int d, void* stream);
fa_status fa_backward_dqdkdv(const void* Q, const void* K, const void* V, const void* dO,
                             const float* workspace, void* dQ, void* dK, void* dV,
                             int B, int H, int N, int d, float scale, int causal, void* stream);
fa_status fa_backward_dkdv(const void* Q, const void* K, const void* V, const void* dO,
                           const float* workspace, void* dK, void* dV,
                           int B, int H, int N, int d, float scale, int causal, void* stream);
fa_status fa_backward_dq(const void* Q, const void* K, const void* V, const void* dO,
                         const float* workspace, void* dQ,
                         int B, int H, int N, int d, float scale, int causal, void* stream);

/* Backward, float32 tensors: same contract as fa_backward, every tensor fp32,
   except that on return the first B*H*N floats of the workspace hold +D. */
fa_status fa_backward_f32(const float* Q, const float* K, const float* V, const float* O,
                          const float* dO, const float* LSE, float* dQ, float* dK, float* dV,
                          float* workspace, int B, int H, int N, int d, float scale, int causal,
                          void* stream);

/* Bytes of workspace fa_backward / fa_backward_f32 need: 8 B H N (0 for invalid sizes). */
size_t fa_backward_workspace_bytes(int B, int H, int N, int d);

/*
 * Decode against a K/V cache, bfloat16 tensors (fp32 accumulation).
 * Page "FlashAttention" (vagrantpi.github.io PKM note), part "⚠️ 注意": in
 * decode each step has a single query token, there is no N x N matrix and
 * the cost is reading K and V; the variant for that case is FlashDecoding.
 * Here the keys of each (batch, head) are split into `splits` contiguous
 * chunks processed in parallel; each chunk yields a normalised partial output
 * O_s and its logsumexp LSE_s (the online softmax of the page's technique 2
 * over the chunk), kept in `workspace`, and a second launch on the same
 * stream combines them:  LSE = log sum_s exp(LSE_s),
 *                        O = sum_s exp(LSE_s - LSE) O_s.
 *
 * Q, O: [B, Nq, H, d] bf16; K, V: [B, Nk, H, d] bf16 (the row layout of the
 * other entry points with N replaced by Nq or Nk); LSE: [B, H, Nq] fp32.
 * causal = 0: every query row sees all Nk keys.  causal = 1: query row i is
 * position Nk - Nq + i of the sequence and sees keys 0 .. Nk - Nq + i
 * (requires Nq <= Nk; Nq = Nk is the square causal forward).
 * splits: 1 .. 4096 key chunks (each holds a whole number of 32-key blocks;
 * chunks past the last key are empty and contribute nothing), or 0 for the
 * library's choice (fa_decode_splits).
 * workspace: caller-owned device memory of fa_decode_workspace_bytes() bytes
 * (4-byte aligned); its contents on return are unspecified.
 * Limits: 1 <= Nq <= 32; Nk as N in the shared limits; d 64 or 128;
 * B*H*chunks <= 2^31 - 1.
 * Errors as for the other entry points, and FA_ERR_INVALID_ARG for Nq <= 0,
 * splits < 0 or (causal = 1 and Nq > Nk); FA_ERR_UNSUPPORTED for Nq > 32 or
 * splits > 4096.
 */
fa_status fa_decode(const void* Q, const void* K, const void* V, void* O, float* LSE,
                    float* workspace, int B, int H, int Nq, int Nk, int d, float scale,
                    int causal, int splits, void* stream);

/* Number of key chunks fa_decode uses when called with splits = 0 (0 for invalid sizes). */
int fa_decode_splits(int B, int H, int Nq, int Nk, int d);

/* Bytes of workspace fa_decode needs: 4 B H S Nq (d + 1) with S the number of
   chunks (splits, or fa_decode_splits() for splits = 0); 0 for invalid sizes. */
size_t fa_decode_workspace_bytes(int B, int H, int Nq, int Nk, int d, int splits);

/*
 * fa_backward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments (minus `workspace`), results (bitwise
 * those of fa_backward) and checks as fa_backward; its 8 B H N bytes of
 * scratch are a static array of the library, 16 MiB on each GPU it runs on,
 * held from the library's first use of that GPU until the process ends.  The
 * call allocates and frees nothing.  Every call on one GPU shares that GPU's
 * array: calls that overlap on one GPU (different streams, or threads without
 * ordering) race and give undefined results.  Nothing in the array needs to be
 * cleared between calls (each call overwrites what it reads).
 * Errors as fa_backward, and FA_ERR_SCRATCH_LIMIT when B*H*N > 2^21 (the
 * array holds two fp32 words per query row); on error nothing is enqueued.
 */
fa_status fa_backward_noalloc(const void* Q, const void* K, const void* V, const void* O,
                              const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                              int B, int H, int N, int d, float scale, int causal, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* fa_status_string(fa_status status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
