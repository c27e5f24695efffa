/*
 * lora_extract.h — recover a rank-r adapter from a weight change (AMD MI355X, gfx950).
 *
 * "two 27B models on a single RTX 5090", TL;DR: comparing the adapted model's
 * weights with the base model's shows a change with the shape of a merged
 * rank-256 LoRA fine-tune, which factored back out is the adapter the serving
 * path applies per request.  The pages do not give the method.  This computes
 * the plainest reading, the truncated singular value decomposition of the
 * change D = W_adapted - W_base = U S V^T:
 *
 *     B = U_r S_r^(1/2)   (N x r),     A = S_r^(1/2) V_r^T   (r x K),     sigma = diag(S_r)
 *
 * so that B A is the best rank-r approximation of D in the Frobenius norm, by
 * the randomized range finder with power iterations (Halko, Martinsson and
 * Tropp, 2011): Omega is the method's K x l random test matrix, drawn by the
 * caller (standard normal entries), l = r + oversampling; power_iters sharpens
 * the range when D's singular values decay slowly.  For a change that is
 * exactly rank r (plus rounding), the result is the truncated SVD to fp32
 * rounding.
 *
 * Layout: W_adapted, W_base device bf16 N x K row-major; omega device fp32
 * K x l row-major; B device fp32 N x r; A device fp32 r x K; sigma device fp32 r
 * (descending).  All 16-byte aligned.  The factors are returned in fp32; round
 * them to bf16 for lora_proj.
 *
 * Limits: 1 <= rank <= l <= min(N, K), l even and at most 512, power_iters
 * 0..8 (else LORA_EUNSUPPORTED); N * K * 4 bytes under 2^36.  workspace: at least
 * lora_extract_workspace_bytes(N, K, l, rank) bytes of device memory, contents
 * not preserved; it must not overlap the inputs or outputs (LORA_EINVAL).
 * Asynchronous on `stream`; the caller owns every buffer.  The eigensolver is
 * one cooperative launch of 64 workgroups.  An extraction of a 5120 x 5120
 * change takes about 20 ms on MI355X, once per weight matrix.
 */
#ifndef LORA_EXTRACT_H
#define LORA_EXTRACT_H

#include "lora_proj.h"

#ifdef __cplusplus
extern "C" {
#endif

lora_status lora_extract(const void* W_adapted, const void* W_base, int64_t N, int64_t K,
                         const float* omega, int32_t l, int32_t rank, int32_t power_iters,
                         float* B, float* A, float* sigma,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes of lora_extract (0 for arguments it would reject). */
size_t lora_extract_workspace_bytes(int64_t N, int64_t K, int32_t l, int32_t rank);

#ifdef __cplusplus
}
#endif

#endif /* LORA_EXTRACT_H */
