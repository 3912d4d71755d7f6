/*
 * gpt_kernels.h -- per-kernel entry points of libgpt.so, for checking each stage of the step
 * on its own.  They run exactly the kernels gpt_fwd_bwd launches, on caller buffers.
 * Conventions as in gpt.h: device pointers, caller-owned memory, stream-ordered, validated
 * before launch, negative status on failure.  `dtype` is GPT_F32 or GPT_BF16 and applies to
 * the arguments marked T; the others are fp32 or int32 as stated.
 */
#ifndef GPT_KERNELS_H_
#define GPT_KERNELS_H_

#include "gpt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C[m,n] (+)= sum_k A(m,k) B(n,k), fp32 C (ldc), T operands.  a_kc/b_kc = 1: element (r,k)
 * at p[r*ld + k]; 0: at p[k*ld + r].  beta 0 overwrites C, 1 adds to it.  K, lda, ldb must be
 * multiples of 8; a row-contiguous A (B) needs M (N) a multiple of 8.  This is the matrix-core
 * GEMM behind every projection of the step (nn.Linear layers of the nanochat GPT class). */
gpt_status gptk_gemm(gpt_dtype dtype, int32_t a_kc, int32_t b_kc, int32_t M, int32_t N, int32_t K,
                     const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                     int64_t ldc, int32_t beta, hipStream_t stream);

/* The weight-gradient form of gptk_gemm (same operands, result and argument rules; N and ldc
 * multiples of 4): bf16 shapes whose output tiling alone would leave compute units idle are
 * split over K, each split writing an fp32 partial [M,N] into `ws`, and the partials are added
 * in split order (deterministic), then written to C or added to it (beta).  ws: caller-owned
 * device fp32 buffer of at least gptk_gemm_wgrad_ws_floats(M, N, K) elements (NULL allowed when
 * that is 0); GPT_EWORKSPACE if it is smaller.  fp32 operands never split. */
gpt_status gptk_gemm_wgrad(gpt_dtype dtype, int32_t a_kc, int32_t b_kc, int32_t M, int32_t N,
                           int32_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                           float* C, int64_t ldc, int32_t beta, float* ws, int64_t ws_floats,
                           hipStream_t stream);
/* fp32 elements of split-K workspace gptk_gemm_wgrad needs for a bf16 M x N x K product. */
int64_t gptk_gemm_wgrad_ws_floats(int32_t M, int32_t N, int32_t K);

/* RMSNorm without weight (`norm` of the nanochat GPT class): x fp32 [N,D] -> y T [N,D],
 * rstd fp32 [N] = 1/sqrt(mean(x^2) + eps).  D a multiple of 64, at most 2048. */
gpt_status gptk_rmsnorm_fwd(gpt_dtype dtype, const float* x, void* y, float* rstd, int64_t N,
                            int32_t D, float eps, hipStream_t stream);

/* dx = dres + rstd * (dy - y * mean(dy * y)), y = x * rstd (dres may be NULL or equal dx);
 * dx_t (T, optional) receives dx rounded to T.  x, rstd, dy, dres, dx fp32. */
gpt_status gptk_rmsnorm_bwd(gpt_dtype dtype, const float* x, const float* rstd, const float* dy,
                            const float* dres, float* dx, void* dx_t, int64_t N, int32_t D,
                            hipStream_t stream);

/* Rotary tables (`_precompute_rotary_embeddings`): cos/sin T [T, hd/2] of t*base^(-2i/hd). */
gpt_status gptk_rope_table(gpt_dtype dtype, void* cos_t, void* sin_t, int32_t T, int32_t hd,
                           float base, hipStream_t stream);

/* In place on the q and k column blocks of qkv T [B*T, 3*H*hd]: half-split rotation
 * (`apply_rotary_emb`) then, if qk_norm, RMSNorm per head; rstd_qk fp32 [B*T, 2H] (q heads
 * then k heads). */
gpt_status gptk_rope_qknorm_fwd(gpt_dtype dtype, void* qkv, const void* cos_t, const void* sin_t,
                                float* rstd_qk, int64_t N, int32_t T, int32_t H, int32_t hd,
                                int32_t qk_norm, float eps, hipStream_t stream);

/* Backward of the above, in place on the dq/dk blocks of dqkv, given the saved qkv output. */
gpt_status gptk_rope_qknorm_bwd(gpt_dtype dtype, void* dqkv, const void* qkv, const void* cos_t,
                                const void* sin_t, const float* rstd_qk, int64_t N, int32_t T,
                                int32_t H, int32_t hd, int32_t qk_norm, hipStream_t stream);

/* The q/k/v projection with rotary + QK-norm in its epilogue (bf16 only), as the bf16 step runs
 * it when H * hd is a multiple of 128: qkv bf16 [N, 3D] = x [N, D] wqkv^T ([3D, D]), then on the
 * q and k blocks the half-split rotation of apply_rotary_emb with the tables of
 * gptk_rope_table (position t = row mod T) and, if qk_norm, RMSNorm per head with rstd_qk
 * fp32 [N, 2H] (q heads then k heads); v columns get u fp32 [N, D] when u is not NULL.  The
 * rotation acts on the fp32 products (the two-kernel form rotates their bf16 rounding). */
gpt_status gptk_qkv_rope_fwd(const void* x, const void* wqkv, void* qkv, const void* cos_t,
                             const void* sin_t, float* rstd_qk, const float* u, int64_t N,
                             int32_t T, int32_t H, int32_t hd, int32_t qk_norm, float eps,
                             hipStream_t stream);

/* Causal attention forward (F.scaled_dot_product_attention(is_causal=True) in the nanochat
 * GPT class): qkv T [B*T, 3D] -> out T [B*T, D], lse2 fp32 [B, H, T] = log2 sum_s
 * 2^(q.k_s * log2(e)/sqrt(hd)) (base-2 log-sum-exp of the scaled scores). */
gpt_status gptk_attention_fwd(gpt_dtype dtype, const void* qkv, void* out, float* lse2, int32_t B,
                              int32_t T, int32_t H, int32_t hd, hipStream_t stream);

/* Attention backward: dqkv T [B*T, 3D] receives dq, dk, dv; scratch fp32 [B*H*T]. */
gpt_status gptk_attention_bwd(gpt_dtype dtype, const void* qkv, const void* out, const void* dout,
                              const float* lse2, float* scratch, void* dqkv, int32_t B,
                              int32_t T, int32_t H, int32_t hd, hipStream_t stream);

/* Softcapped cross-entropy forward + backward in place (GPT.forward's loss): z T [rows, V]
 * (row stride ldz) is overwritten by dz = (softmax(c) - onehot) (1 - tanh^2(z/cap))
 * * grad_scale / n_valid, c = cap tanh(z/cap) (cap 0: c = z); loss_rows fp32 [rows] gets
 * logsumexp(c) - c[target] (0 for ignored targets).  n_valid: int32 device scalar.
 * V a multiple of 64, at most 65536. */
gpt_status gptk_softcap_ce(gpt_dtype dtype, void* z, int64_t ldz, const int32_t* targets,
                           int64_t rows, int32_t V, float cap, float grad_scale,
                           const int32_t* n_valid, float* loss_rows, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* GPT_KERNELS_H_ */
