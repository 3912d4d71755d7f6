// Softcapped cross-entropy forward + backward over bf16/fp32 logits (GPT.forward on the
// nanochat page: logits = 15 tanh(logits / 15), float cross-entropy with ignore_index -1,
// mean reduction).  One workgroup owns one token row: it reads the row once into registers,
// reduces the maximum and the sum of exponentials, and overwrites the row in place with
//   dz = (softmax(c) - onehot(target)) * (1 - tanh^2(z / cap)) * grad_scale / n_valid,
// so full-precision logits never exist in memory.  The per-row losses are summed in a fixed
// order by a single workgroup (deterministic).
#include "kernels.h"

namespace gpt {
namespace {

__global__ void count_targets_kernel(const int32_t* __restrict__ tgt, long long N, int V,
                                     int* __restrict__ n_valid, int* err) {
  __shared__ int total;
  if (threadIdx.x == 0) total = 0;
  __syncthreads();
  int c = 0, bad = 0;
  for (long long i = threadIdx.x; i < N; i += blockDim.x) {
    const int t = tgt[i];
    if (t >= 0 && t < V) ++c;
    else if (t != -1) bad = 1;
  }
  atomicAdd(&total, c);
  if (bad) atomicOr(err, 2);
  __syncthreads();
  if (threadIdx.x == 0) *n_valid = total;
}

constexpr float LOG2E = 1.4426950408889634f;

// 2^x and 1/x with the hardware instructions (v_exp_f32, v_rcp_f32: about 1 ulp).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

typedef __fp16 h2 __attribute__((ext_vector_type(2)));

// Per-thread storage of exp(c - thread max): packed fp16 pairs for bf16 logits (the value is in
// (0, 1]; fp16 keeps 11 bits, more than the bf16 gradient that is stored from it), fp32 pairs for
// fp32 logits.
template <typename T> struct EStore;
template <> struct EStore<bf16> {
  h2 v;
  __device__ __forceinline__ void set(float a, float b) { v = __builtin_amdgcn_cvt_pkrtz(a, b); }
  __device__ __forceinline__ float get(int i) const { return (float)v[i]; }
};
template <> struct EStore<float> {
  float v[2];
  __device__ __forceinline__ void set(float a, float b) { v[0] = a; v[1] = b; }
  __device__ __forceinline__ float get(int i) const { return v[i]; }
};

// One workgroup per token row; thread-local pieces of 8 columns (at most G per thread).  The row
// is read once into registers as th = tanh(z / cap) (or z without a cap); each thread then forms
// e = exp(c - m_t) with its own maximum m_t (c = cap * th) and their sum s_t, and the block
// combines M = max m_t and S = sum s_t exp(m_t - M), so lse = M + ln S.  The gradient needs no
// further exponential: p = e * exp(m_t - M) / S, and only the lane that owns the target column
// subtracts the one-hot term.
template <typename T, int CE_THREADS, int G, bool CAPPED>
__device__ __forceinline__ void ce_row(T* __restrict__ z, long long ldz,
                                       const int32_t* __restrict__ tgt, int V, float cap,
                                       float grad_scale, const int* __restrict__ n_valid,
                                       float* __restrict__ loss_rows, float* smem) {
  const long long row = blockIdx.x;
  T* zr = z + row * ldz;
  const int groups = V / 8;
  const int t = tgt[row];
  const bool valid = t >= 0 && t < V;
  constexpr bool capped = CAPPED;
  const float k2 = capped ? 2.f * LOG2E / cap : 0.f;  // exp(2 z / cap) = 2^(z * k2)
  float th[G][8];
  EStore<T> ev[G][4];
  float mt = -INFINITY;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int g = threadIdx.x + gi * CE_THREADS;
    if (g < groups) {
      load8_f32(zr + g * 8, th[gi]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (capped) th[gi][e] = 1.f - 2.f * hw_rcp(hw_exp2(th[gi][e] * k2) + 1.f);
        mt = fmaxf(mt, capped ? cap * th[gi][e] : th[gi][e]);
      }
    }
  }
  const float cmul = capped ? cap : 1.f;
  float st = 0.f;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int g = threadIdx.x + gi * CE_THREADS;
    if (g < groups) {
      float ex[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ex[e] = hw_exp2((cmul * th[gi][e] - mt) * LOG2E);
        st += ex[e];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) ev[gi][q].set(ex[2 * q], ex[2 * q + 1]);
    }
  }
  const float M = block_max(mt, smem);
  const float S = block_sum(st * hw_exp2((mt - M) * LOG2E), smem);
  const float lse = M + __logf(S);
  const int nv = *n_valid;
  const float scale = valid ? grad_scale / (float)(nv > 0 ? nv : 1) : 0.f;
  const float f = hw_exp2((mt - M) * LOG2E) / S * scale;  // e * f = softmax * scale
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int g = threadIdx.x + gi * CE_THREADS;
    if (g < groups) {
      float d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = ev[gi][e / 2].get(e % 2) * f;
        d[e] = capped ? p * fmaf(-th[gi][e], th[gi][e], 1.f) : p;
      }
      if (valid && g == t / 8) {  // the target column: one lane of the row
        const int e = t % 8;
        float c = 0.f, dt = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q == e) {
            c = cmul * th[gi][q];
            dt = capped ? fmaf(-th[gi][q], th[gi][q], 1.f) : 1.f;
          }
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q == e) d[q] -= scale * dt;
        loss_rows[row] = lse - c;
      }
      store8_f32(zr + g * 8, d);
    }
  }
  if (!valid && threadIdx.x == 0) loss_rows[row] = 0.f;
}

// CAPPED: cap > 0 (chosen on the host, so each kernel holds one of the two row bodies)
template <typename T, int CE_THREADS, int G, bool CAPPED>
__global__ __launch_bounds__(CE_THREADS) void ce_kernel(T* __restrict__ z, long long ldz,
                                                        const int32_t* __restrict__ tgt, int V,
                                                        float cap, float grad_scale,
                                                        const int* __restrict__ n_valid,
                                                        float* __restrict__ loss_rows) {
  __shared__ float smem[16];
  ce_row<T, CE_THREADS, G, CAPPED>(z, ldz, tgt, V, cap, grad_scale, n_valid, loss_rows, smem);
}

__global__ void loss_reduce_kernel(const float* __restrict__ loss_rows, long long N,
                                   const int* __restrict__ n_valid, float* __restrict__ loss) {
  __shared__ float smem[16];
  float s = 0.f;
  for (long long i = threadIdx.x; i < N; i += blockDim.x) s += loss_rows[i];
  s = block_sum(s, smem);
  if (threadIdx.x == 0) {
    const int nv = *n_valid;
    *loss = s / (float)(nv > 0 ? nv : 1);
  }
}

}  // namespace

gpt_status launch_count_targets(const int32_t* tgt, long long N, int V, int* n_valid, int* err,
                                hipStream_t s) {
  count_targets_kernel<<<1, 1024, 0, s>>>(tgt, N, V, n_valid, err);
  return check_launch("count targets");
}

template <typename T>
gpt_status launch_ce(T* z, long long ldz, const int32_t* tgt, long long rows, int V, float cap,
                     float grad_scale, const int* n_valid, float* loss_rows, hipStream_t s) {
  if (rows == 0) return GPT_OK;
  // Each of the row's V/8 vectors lives in one thread's registers (at most 8 per thread).
  const int g = V / 8;
#define CE_CASE(TH, G)                                                                         \
  (cap > 0.f ? ce_kernel<T, TH, G, true><<<(unsigned)rows, TH, 0, s>>>(                         \
                   z, ldz, tgt, V, cap, grad_scale, n_valid, loss_rows)                         \
             : ce_kernel<T, TH, G, false><<<(unsigned)rows, TH, 0, s>>>(                        \
                   z, ldz, tgt, V, cap, grad_scale, n_valid, loss_rows))
  // (16 pieces of 8 in 512 threads for the large softcapped vocabularies: two waves per SIMD with
  // room for the row's 128 tanh values and 64 packed exponentials per lane; without a cap the
  // 1024-thread form fits its registers)
  if (g <= 256) CE_CASE(256, 1);
  else if (g <= 1024) CE_CASE(256, 4);
  else if (g <= 2048) CE_CASE(256, 8);
  else if (g <= 4096) CE_CASE(512, 8);
  else if (g <= 8192 && cap > 0.f) CE_CASE(512, 16);
  else if (g <= 8192) CE_CASE(1024, 8);
  else return fail(GPT_ESHAPE, "vocab above 65536 is not supported");
#undef CE_CASE
  return check_launch("cross-entropy");
}

gpt_status launch_loss_reduce(const float* loss_rows, long long N, const int* n_valid,
                              float* loss, hipStream_t s) {
  loss_reduce_kernel<<<1, 1024, 0, s>>>(loss_rows, N, n_valid, loss);
  return check_launch("loss reduce");
}

template gpt_status launch_ce<float>(float*, long long, const int32_t*, long long, int, float,
                                     float, const int*, float*, hipStream_t);
template gpt_status launch_ce<bf16>(bf16*, long long, const int32_t*, long long, int, float,
                                    float, const int*, float*, hipStream_t);

}  // namespace gpt
