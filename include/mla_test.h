/*
 * mla_test.h -- measurement and step-parity entry points of the MLA library (not part of the
 * layer API in mla.h; same status codes, ownership and validation rules).
 */
#ifndef MLA_TEST_H_
#define MLA_TEST_H_

#include "mla.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Stage names of mla_test_gemm: which projection's kernel symbol the launch uses (the code is
 * identical; the symbol lets traces attribute time to a stage). */
enum {
  MLA_STAGE_NONE = 0, MLA_STAGE_QKVA = 1, MLA_STAGE_QB = 2, MLA_STAGE_KVB = 3, MLA_STAGE_OPROJ = 4,
  MLA_STAGE_ABSORB = 5, MLA_STAGE_UV = 6, MLA_STAGE_DECODE_ATTN = 7, MLA_STAGE_PREFILL_ATTN = 8
};

/* Stage probe for measurement: arms a one-shot probe on the calling thread. The next layer call
 * (prefill, decode, their block and static forms) made from this thread that launches `stage`
 * records ev_before (a hipEvent_t) on the call's stream right before that stage's launches and
 * ev_after right after them, then disarms; their elapsed time is the stage's duration on the
 * stream. Stages: MLA_STAGE_OPROJ (o_proj with its split-K reduction, if any),
 * MLA_STAGE_DECODE_ATTN (the split attention over the latent cache, without the merge),
 * MLA_STAGE_PREFILL_ATTN (causal prefill attention); MLA_STAGE_NONE disarms. The events are the
 * caller's and must stay valid until the call has been enqueued. MLA_E_ARG for another stage or
 * a NULL event. */
mla_status mla_test_probe_stage(int32_t stage, void* ev_before, void* ev_after);

/* Workspace bytes mla_test_gemm needs for this shape (split-K partials). */
size_t mla_test_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K, int32_t batch);

/* The projection kernel on its own: for b < batch, C[b] = A[b] B[b]^T, i.e. y = x W^T of an
 * nn.Linear without bias whose weight is [out, in] ("Key-value latent" page, mla-init excerpt;
 * attention_bias is false in the config). A [M, K] (row stride lda, batch stride sA) and
 * B [N, K] (ldb, sB) are device bf16; C [M, N] (ldc, sC) is device float32 (out_bf16 = 0) or
 * bf16 (out_bf16 = 1); strides in elements. K must be a multiple of 128, lda/ldb multiples of 8.
 * ws: device workspace of ws_bytes >= mla_test_gemm_workspace_bytes() (scratch only). The same kernels and launch plan as the layer's projections are used. */
mla_status mla_test_gemm(int32_t M, int32_t N, int32_t K, int32_t batch, const void* A, int64_t lda, int64_t sA,
                         const void* B, int64_t ldb, int64_t sB, void* C, int64_t ldc, int64_t sC, int32_t out_bf16,
                         int32_t stage, void* ws, size_t ws_bytes, mla_stream stream);

/* Workspace bytes mla_test_gemm_fp8 needs for this shape (split-K partials). */
size_t mla_test_gemm_fp8_workspace_bytes(int32_t M, int32_t N, int32_t K);

/* The FP8 projection kernel on its own ("Key-value latent" page, linear excerpt: E4M3 weights with
 * one scale per 128 x 128 block, activations quantised per token and 128 features):
 * C[m][n] = sum_k (a[m][k] * a_scale[m][k/128]) * (b[n][k] * b_scale[n/128][k/128]).
 * A [M, K] and B [N, K] are device E4M3FN codes, rows K bytes apart; a_scale [M][K/128] and
 * b_scale [ceil(N/128)][K/128] device float32, rows K/128 apart; C [M, N] device float32, rows N
 * apart. precise = 1: the form of q_a|kv_a and kv_b (codes widened exactly to bf16, each 128-wide
 * group summed by bf16 MFMAs into float32); precise = 0: the form of q_b and o_proj (one FP8 MFMA
 * per group with unit hardware scales). K must be a multiple of 128, N of 8. ws: device workspace of
 * ws_bytes >= mla_test_gemm_fp8_workspace_bytes() (scratch only). */
mla_status mla_test_gemm_fp8(int32_t M, int32_t N, int32_t K, const void* A, const float* a_scale, const void* B,
                             const float* b_scale, float* C, int32_t precise, void* ws, size_t ws_bytes,
                             mla_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_TEST_H_ */
