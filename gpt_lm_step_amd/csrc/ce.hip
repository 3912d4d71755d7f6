// Softcapped cross-entropy forward + backward over bf16/fp32 logits (GPT.forward on the
// nanochat page: logits = 15 tanh(logits / 15), float cross-entropy with ignore_index -1,
// mean reduction).  One workgroup owns one token row: it reads the row once into registers,
// reduces max and sum of exp, and overwrites the row in place with
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

// tanh(x) = 1 - 2 / (exp(2x) + 1): exact limits at +-inf, |error| ~ 1e-7.
__device__ __forceinline__ float fast_tanh(float x) {
  return 1.f - 2.f / (__expf(2.f * x) + 1.f);
}

template <typename T, int CE_THREADS, int G>
__global__ __launch_bounds__(CE_THREADS) void ce_kernel(T* __restrict__ z, long long ldz,
                                                        const int32_t* __restrict__ tgt, int V,
                                                        float cap, float grad_scale,
                                                        const int* __restrict__ n_valid,
                                                        float* __restrict__ loss_rows) {
  __shared__ float smem[16];
  const long long row = blockIdx.x;
  T* zr = z + row * ldz;
  const int groups = V / 8;
  const int t = tgt[row];
  const bool valid = t >= 0 && t < V;
  const float inv_cap = cap > 0.f ? 1.f / cap : 0.f;
  float c[G][8];
  float mx = -INFINITY;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int g = threadIdx.x + gi * CE_THREADS;
    if (g < groups) {
      load8_f32(zr + g * 8, c[gi]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (cap > 0.f) c[gi][e] = cap * fast_tanh(c[gi][e] * inv_cap);
        mx = fmaxf(mx, c[gi][e]);
      }
    }
  }
  mx = block_max(mx, smem);
  float se = 0.f;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int g = threadIdx.x + gi * CE_THREADS;
    if (g < groups) {
#pragma unroll
      for (int e = 0; e < 8; ++e) se += __expf(c[gi][e] - mx);
    }
  }
  se = block_sum(se, smem);
  const float lse = mx + __logf(se);
  const int nv = *n_valid;
  const float scale = valid ? grad_scale / (float)(nv > 0 ? nv : 1) : 0.f;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int g = threadIdx.x + gi * CE_THREADS;
    if (g < groups) {
      float d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int col = g * 8 + e;
        const float p = __expf(c[gi][e] - lse);
        float gr = p - (col == t ? 1.f : 0.f);
        if (cap > 0.f) {
          const float th = c[gi][e] * inv_cap;
          gr *= 1.f - th * th;
        }
        d[e] = gr * scale;
        if (col == t) loss_rows[row] = lse - c[gi][e];
      }
      store8_f32(zr + g * 8, d);
    }
  }
  if (!valid && threadIdx.x == 0) loss_rows[row] = 0.f;
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
#define CE_CASE(TH, G)                                                                          \
  ce_kernel<T, TH, G><<<(unsigned)rows, TH, 0, s>>>(z, ldz, tgt, V, cap, grad_scale, n_valid, \
                                                    loss_rows)
  if (g <= 256) CE_CASE(256, 1);
  else if (g <= 1024) CE_CASE(256, 4);
  else if (g <= 2048) CE_CASE(256, 8);
  else if (g <= 4096) CE_CASE(512, 8);
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
