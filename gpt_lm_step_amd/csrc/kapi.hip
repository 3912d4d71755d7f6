// Per-kernel entry points (include/gpt_kernels.h): validation, then the same launchers the
// step uses.
#include "../../include/gpt_kernels.h"
#include "gemm.h"

using namespace gpt;

namespace {
bool bad_dtype(int32_t d) { return d != GPT_F32 && d != GPT_BF16; }
}

extern "C" {

gpt_status gptk_gemm(gpt_dtype dtype, int32_t a_kc, int32_t b_kc, int32_t M, int32_t N, int32_t K,
                     const void* A, int64_t lda, const void* B, int64_t ldb, float* C,
                     int64_t ldc, int32_t beta, hipStream_t stream) {
  if (bad_dtype(dtype) || !A || !B || !C) return fail(GPT_EINVAL, "gptk_gemm: bad dtype or null");
  if (M < 0 || N < 0 || K < 0 || ldc < N || ldc % 4) return fail(GPT_ESHAPE, "gptk_gemm: bad sizes");
  if (((uintptr_t)C) % 16) return fail(GPT_EINVAL, "gptk_gemm: C must be 16-byte aligned");
  EpiStoreF32 epi{C, ldc, beta ? 1 : 0};
  if (dtype == GPT_BF16)
    return gemm<G_TEST, bf16>(a_kc, b_kc, M, N, K, (const bf16*)A, lda, (const bf16*)B, ldb, epi, stream);
  return gemm<G_TEST, float>(a_kc, b_kc, M, N, K, (const float*)A, lda, (const float*)B, ldb, epi, stream);
}

gpt_status gptk_gemm_wgrad(gpt_dtype dtype, int32_t a_kc, int32_t b_kc, int32_t M, int32_t N,
                           int32_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                           float* C, int64_t ldc, int32_t beta, float* ws, int64_t ws_floats,
                           hipStream_t stream) {
  if (bad_dtype(dtype) || !A || !B || !C) return fail(GPT_EINVAL, "gptk_gemm_wgrad: bad dtype or null");
  if (M < 0 || N < 0 || K < 0 || ldc < N || ldc % 4) return fail(GPT_ESHAPE, "gptk_gemm_wgrad: bad sizes");
  if (((uintptr_t)C) % 16) return fail(GPT_EINVAL, "gptk_gemm_wgrad: C must be 16-byte aligned");
  if (ws_floats < 0) return fail(GPT_EINVAL, "gptk_gemm_wgrad: negative workspace size");
  EpiStoreF32 epi{C, ldc, beta ? 1 : 0};
  if (dtype == GPT_BF16)
    return gemm_wgrad<G_TEST, bf16>(a_kc, b_kc, M, N, K, (const bf16*)A, lda, (const bf16*)B, ldb,
                                    epi, ws, ws_floats, stream);
  return gemm_wgrad<G_TEST, float>(a_kc, b_kc, M, N, K, (const float*)A, lda, (const float*)B,
                                   ldb, epi, ws, ws_floats, stream);
}

int64_t gptk_gemm_wgrad_ws_floats(int32_t M, int32_t N, int32_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return gemm_wgrad_ws_floats(M, N, K);
}

gpt_status gptk_rmsnorm_fwd(gpt_dtype dtype, const float* x, void* y, float* rstd, int64_t N,
                            int32_t D, float eps, hipStream_t stream) {
  if (bad_dtype(dtype) || !x || !y || !rstd) return fail(GPT_EINVAL, "gptk_rmsnorm_fwd: null");
  if (N < 0 || D <= 0 || D % 64 || D > 2048) return fail(GPT_ESHAPE, "gptk_rmsnorm_fwd: bad D");
  if (N == 0) return GPT_OK;
  if (dtype == GPT_BF16) return launch_rms_fwd<bf16>(x, (bf16*)y, rstd, N, D, eps, stream);
  return launch_rms_fwd<float>(x, (float*)y, rstd, N, D, eps, stream);
}

gpt_status gptk_rmsnorm_bwd(gpt_dtype dtype, const float* x, const float* rstd, const float* dy,
                            const float* dres, float* dx, void* dx_t, int64_t N, int32_t D,
                            hipStream_t stream) {
  if (bad_dtype(dtype) || !x || !rstd || !dy || !dx) return fail(GPT_EINVAL, "gptk_rmsnorm_bwd: null");
  if (N < 0 || D <= 0 || D % 64 || D > 2048) return fail(GPT_ESHAPE, "gptk_rmsnorm_bwd: bad D");
  if (N == 0) return GPT_OK;
  if (dtype == GPT_BF16)
    return launch_rms_bwd<bf16>(x, rstd, dy, dres, dx, (bf16*)dx_t, N, D, stream);
  return launch_rms_bwd<float>(x, rstd, dy, dres, dx, (float*)dx_t, N, D, stream);
}

gpt_status gptk_rope_table(gpt_dtype dtype, void* cos_t, void* sin_t, int32_t T, int32_t hd,
                           float base, hipStream_t stream) {
  if (bad_dtype(dtype) || !cos_t || !sin_t) return fail(GPT_EINVAL, "gptk_rope_table: null");
  if (T <= 0 || hd <= 0 || hd % 2) return fail(GPT_ESHAPE, "gptk_rope_table: bad sizes");
  if (dtype == GPT_BF16) return launch_rope_table<bf16>((bf16*)cos_t, (bf16*)sin_t, T, hd, base, stream);
  return launch_rope_table<float>((float*)cos_t, (float*)sin_t, T, hd, base, stream);
}

static gpt_status check_heads(int64_t N, int32_t T, int32_t H, int32_t hd) {
  if (T <= 0 || H <= 0 || N < 0 || N % T) return fail(GPT_ESHAPE, "bad N, T or H");
  if (hd != 32 && hd != 64 && hd != 128) return fail(GPT_ESHAPE, "head_dim must be 32, 64 or 128");
  return GPT_OK;
}

gpt_status gptk_rope_qknorm_fwd(gpt_dtype dtype, void* qkv, const void* cos_t, const void* sin_t,
                                float* rstd_qk, int64_t N, int32_t T, int32_t H, int32_t hd,
                                int32_t qk_norm, float eps, hipStream_t stream) {
  if (bad_dtype(dtype) || !qkv || !cos_t || !sin_t || !rstd_qk) return fail(GPT_EINVAL, "gptk_rope_qknorm_fwd: null");
  gpt_status st = check_heads(N, T, H, hd);
  if (st != GPT_OK || N == 0) return st;
  if (dtype == GPT_BF16)
    return launch_rope_qknorm_fwd<bf16>((bf16*)qkv, (const bf16*)cos_t, (const bf16*)sin_t,
                                        rstd_qk, N, T, H, hd, qk_norm, eps, stream);
  return launch_rope_qknorm_fwd<float>((float*)qkv, (const float*)cos_t, (const float*)sin_t,
                                       rstd_qk, N, T, H, hd, qk_norm, eps, stream);
}

gpt_status gptk_rope_qknorm_bwd(gpt_dtype dtype, void* dqkv, const void* qkv, const void* cos_t,
                                const void* sin_t, const float* rstd_qk, int64_t N, int32_t T,
                                int32_t H, int32_t hd, int32_t qk_norm, hipStream_t stream) {
  if (bad_dtype(dtype) || !dqkv || !qkv || !cos_t || !sin_t || !rstd_qk)
    return fail(GPT_EINVAL, "gptk_rope_qknorm_bwd: null");
  gpt_status st = check_heads(N, T, H, hd);
  if (st != GPT_OK || N == 0) return st;
  if (dtype == GPT_BF16)
    return launch_rope_qknorm_bwd<bf16>((bf16*)dqkv, (const bf16*)qkv, (const bf16*)cos_t,
                                        (const bf16*)sin_t, rstd_qk, N, T, H, hd, qk_norm, stream);
  return launch_rope_qknorm_bwd<float>((float*)dqkv, (const float*)qkv, (const float*)cos_t,
                                       (const float*)sin_t, rstd_qk, N, T, H, hd, qk_norm, stream);
}

gpt_status gptk_qkv_rope_fwd(const void* x, const void* wqkv, void* qkv, const void* cos_t,
                             const void* sin_t, float* rstd_qk, const float* u, int64_t N,
                             int32_t T, int32_t H, int32_t hd, int32_t qk_norm, float eps,
                             hipStream_t stream) {
  if (!x || !wqkv || !qkv || !cos_t || !sin_t || !rstd_qk)
    return fail(GPT_EINVAL, "gptk_qkv_rope_fwd: null");
  gpt_status st = check_heads(N, T, H, hd);
  if (st != GPT_OK || N == 0) return st;
  const int D = H * hd;
  if (D % 128) return fail(GPT_ESHAPE, "gptk_qkv_rope_fwd: H * hd must be a multiple of 128");
  if (((uintptr_t)qkv | (uintptr_t)u) % 16) return fail(GPT_EINVAL, "gptk_qkv_rope_fwd: misaligned");
  auto go = [&](auto qkn_c, auto vadd_c) {
    constexpr bool QKN = decltype(qkn_c)::value, VADD = decltype(vadd_c)::value;
    const EpiQKVRope<bf16, QKN, VADD> e{(bf16*)qkv, 3LL * D, (const bf16*)cos_t,
                                        (const bf16*)sin_t, rstd_qk, u, D, D, hd, T, H, eps};
    return gemm<G_TEST, bf16>(true, true, (int)N, 3 * D, D, (const bf16*)x, D,
                              (const bf16*)wqkv, D, e, stream);
  };
  if (qk_norm) return u ? go(std::true_type(), std::true_type()) : go(std::true_type(), std::false_type());
  return u ? go(std::false_type(), std::true_type()) : go(std::false_type(), std::false_type());
}

gpt_status gptk_attention_fwd(gpt_dtype dtype, const void* qkv, void* out, float* lse2, int32_t B,
                              int32_t T, int32_t H, int32_t hd, hipStream_t stream) {
  if (bad_dtype(dtype) || !qkv || !out || !lse2) return fail(GPT_EINVAL, "gptk_attention_fwd: null");
  if (B <= 0 || T <= 0 || T % 64) return fail(GPT_ESHAPE, "gptk_attention_fwd: T must be a multiple of 64");
  gpt_status st = check_heads((int64_t)B * T, T, H, hd);
  if (st != GPT_OK) return st;
  if (dtype == GPT_BF16)
    return launch_attn_fwd<bf16>((const bf16*)qkv, (bf16*)out, lse2, B, T, H, hd, stream);
  return launch_attn_fwd<float>((const float*)qkv, (float*)out, lse2, B, T, H, hd, stream);
}

gpt_status gptk_attention_bwd(gpt_dtype dtype, const void* qkv, const void* out, const void* dout,
                              const float* lse2, float* scratch, void* dqkv, int32_t B,
                              int32_t T, int32_t H, int32_t hd, hipStream_t stream) {
  if (bad_dtype(dtype) || !qkv || !out || !dout || !lse2 || !scratch || !dqkv)
    return fail(GPT_EINVAL, "gptk_attention_bwd: null");
  if (B <= 0 || T <= 0 || T % 64) return fail(GPT_ESHAPE, "gptk_attention_bwd: T must be a multiple of 64");
  gpt_status st = check_heads((int64_t)B * T, T, H, hd);
  if (st != GPT_OK) return st;
  if (dtype == GPT_BF16)
    return launch_attn_bwd<bf16>((const bf16*)qkv, (const bf16*)out, (const bf16*)dout, lse2,
                                 scratch, (bf16*)dqkv, B, T, H, hd, stream);
  return launch_attn_bwd<float>((const float*)qkv, (const float*)out, (const float*)dout, lse2,
                                scratch, (float*)dqkv, B, T, H, hd, stream);
}

gpt_status gptk_softcap_ce(gpt_dtype dtype, void* z, int64_t ldz, const int32_t* targets,
                           int64_t rows, int32_t V, float cap, float grad_scale,
                           const int32_t* n_valid, float* loss_rows, hipStream_t stream) {
  if (bad_dtype(dtype) || !z || !targets || !n_valid || !loss_rows)
    return fail(GPT_EINVAL, "gptk_softcap_ce: null");
  if (rows < 0 || V <= 0 || V % 64 || V > 65536 || ldz < V || ldz % 8)
    return fail(GPT_ESHAPE, "gptk_softcap_ce: bad sizes");
  if (dtype == GPT_BF16)
    return launch_ce<bf16>((bf16*)z, ldz, targets, rows, V, cap, grad_scale, n_valid, loss_rows, stream);
  return launch_ce<float>((float*)z, ldz, targets, rows, V, cap, grad_scale, n_valid, loss_rows, stream);
}

}  // extern "C"
