// The dense optimizer step that follows a training step: the training script of the "$1000 tier
// nanochat run" discussion (nanochat #8) clips the global gradient norm in its accumulation loop,
// steps the token embedding and the LM head with Adam and every matrix of the blocks with Muon
// (the `Muon` class and `zeropower_via_newtonschulz5`); the modded-nanogpt README runs the
// Newton-Schulz iteration in bfloat16.
//
// Muon matrices are stepped in batches of one shape: the D x D blocks (q, k, v and the output
// projection of every layer, four consecutive D*D blocks per layer), the MLP up projections
// [F, D] and the MLP down projections [D, F] (and the trigram projection).  Each Newton-Schulz
// step is three batched bf16 GEMMs on the matrix cores (fp32 accumulation, one rounding per new
// matrix); tall matrices are handled through the operand layouts instead of transposed copies.
#include <math.h>

#include <algorithm>

#include "gemm.h"

namespace gpt {
namespace {

constexpr int OPT_THREADS = 256;
constexpr int NORM_PARTS = 1024;  // fixed partial count: the same summation order on every device
constexpr float NS_A = 3.4445f, NS_B = -4.7750f, NS_C = 2.0315f;

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
// Sum over the block in a fixed order (thread 0 gets it).
__device__ __forceinline__ double block_sum_d(double v, double* sm) {
  v = wave_sum_d(v);
  const int w = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  if (threadIdx.x % WAVE == 0) sm[w] = v;
  __syncthreads();
  double t = 0;
  for (int i = 0; i < nw; ++i) t += sm[i];
  return t;
}

// part[b] = sum of g^2 over the b-th of NORM_PARTS contiguous chunks of [0, n) (n % 4 == 0).
__global__ __launch_bounds__(OPT_THREADS) void sumsq_kernel(const float* __restrict__ g, long long n,
                                                             double* __restrict__ part) {
  __shared__ double sm[OPT_THREADS / WAVE];
  const long long per = ((n + NORM_PARTS - 1) / NORM_PARTS + 3) / 4 * 4;
  const long long lo = min(n, (long long)blockIdx.x * per), hi = min(n, lo + per);
  double acc = 0;
  for (long long i = lo + 4LL * threadIdx.x; i < hi; i += 4LL * OPT_THREADS) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(g + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc += (double)v[e] * v[e];
  }
  const double t = block_sum_d(acc, sm);
  if (threadIdx.x == 0) part[blockIdx.x] = t;
}

// Global norm and clip factor: scal[0] = min(1, clip / (norm + 1e-6)) (1 without clipping),
// scal[1] = norm; norm_out (may be null) receives the norm too.
__global__ __launch_bounds__(NORM_PARTS) void clip_factor_kernel(const double* __restrict__ part,
                                                                 float clip, float* __restrict__ scal,
                                                                 float* __restrict__ norm_out) {
  __shared__ double sm[NORM_PARTS / WAVE];
  const double t = block_sum_d(part[threadIdx.x], sm);
  if (threadIdx.x == 0) {
    const double norm = sqrt(t);
    const double f = clip > 0.f ? fmin(1.0, (double)clip / (norm + 1e-6)) : 1.0;
    scal[0] = (float)f;
    scal[1] = (float)norm;
    if (norm_out) *norm_out = (float)norm;
  }
}

template <typename T>
__device__ __forceinline__ void store4_opt(T* p, const float (&v)[4]) {
  vec4t<T> o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = from_f32<T>(v[i]);
  *reinterpret_cast<vec4t<T>*>(p) = o;
}

// Bias-corrected Adam with decoupled weight decay over [0, n) (n % 4 == 0); g is scaled by the
// clip factor; copy (may be null) receives the new weights in T.
template <typename T>
__global__ __launch_bounds__(OPT_THREADS) void adam_kernel(
    float* __restrict__ p, T* __restrict__ copy, const float* __restrict__ g, float* __restrict__ m,
    float* __restrict__ v, long long n, const float* __restrict__ scal, float lr, float beta1,
    float beta2, float step_size, float inv_sqrt_bc2, float eps, float wd) {
  const float f = scal[0];
  for (long long i = 4LL * ((long long)blockIdx.x * OPT_THREADS + threadIdx.x); i < n;
       i += 4LL * OPT_THREADS * gridDim.x) {
    const f32x4 gv = *reinterpret_cast<const f32x4*>(g + i);
    f32x4 pv = *reinterpret_cast<const f32x4*>(p + i);
    f32x4 mv = *reinterpret_cast<const f32x4*>(m + i);
    f32x4 vv = *reinterpret_cast<const f32x4*>(v + i);
    float out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gi = gv[e] * f;
      mv[e] += (1.f - beta1) * (gi - mv[e]);
      vv[e] = beta2 * vv[e] + (1.f - beta2) * gi * gi;
      const float denom = sqrtf(vv[e]) * inv_sqrt_bc2 + eps;
      pv[e] = pv[e] * (1.f - lr * wd) - step_size * mv[e] / denom;
      out[e] = pv[e];
    }
    *reinterpret_cast<f32x4*>(p + i) = pv;
    *reinterpret_cast<f32x4*>(m + i) = mv;
    *reinterpret_cast<f32x4*>(v + i) = vv;
    if (copy) store4_opt(copy + i, out);
  }
}

// A batch of equally shaped matrices inside the flat buffers: matrix z starts at
// base + (z / per_layer) * layer_stride + (z % per_layer) * sub_stride.
struct MatGroup {
  long long base, layer_stride, sub_stride;
  int per_layer, count, rows, cols;
};
__device__ __forceinline__ long long mat_off(const MatGroup& G, int z) {
  return G.base + (long long)(z / G.per_layer) * G.layer_stride +
         (long long)(z % G.per_layer) * G.sub_stride;
}

// Momentum of matrix z = blockIdx.y, chunk blockIdx.x of gridDim.x: buf += (1 - mu)(g - buf),
// u = g + mu (buf - g) (Nesterov) or buf; X = bf16(u) in the matrix's layout; part[z][chunk] =
// sum of bf16(u)^2.
__global__ __launch_bounds__(OPT_THREADS) void muon_momentum_kernel(
    const float* __restrict__ g, float* __restrict__ mom, bf16* __restrict__ X,
    double* __restrict__ part, MatGroup G, const float* __restrict__ scal, float mu, int nesterov) {
  __shared__ double sm[OPT_THREADS / WAVE];
  const int z = blockIdx.y;
  const long long n = (long long)G.rows * G.cols, off = mat_off(G, z);
  const long long per = ((n + gridDim.x - 1) / gridDim.x + 3) / 4 * 4;
  const long long lo = min(n, (long long)blockIdx.x * per), hi = min(n, lo + per);
  const float f = scal[0];
  double acc = 0;
  for (long long i = lo + 4LL * threadIdx.x; i < hi; i += 4LL * OPT_THREADS) {
    const f32x4 gv = *reinterpret_cast<const f32x4*>(g + off + i);
    f32x4 bv = *reinterpret_cast<const f32x4*>(mom + off + i);
    float u[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float gi = gv[e] * f;
      bv[e] += (1.f - mu) * (gi - bv[e]);
      u[e] = nesterov ? gi + mu * (bv[e] - gi) : bv[e];
    }
    *reinterpret_cast<f32x4*>(mom + off + i) = bv;
    bf16x4 xb;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xb[e] = (bf16)u[e];
      const double x = (double)(float)xb[e];
      acc += x * x;
    }
    *reinterpret_cast<bf16x4*>(X + (long long)z * n + i) = xb;
  }
  const double t = block_sum_d(acc, sm);
  if (threadIdx.x == 0) part[(long long)z * gridDim.x + blockIdx.x] = t;
}

// X_z = bf16(X_z / (||X_z||_F + 1e-7)), the norm from matrix z's nparts partial sums.
__global__ __launch_bounds__(OPT_THREADS) void ns_scale_kernel(bf16* __restrict__ X,
                                                               const double* __restrict__ part,
                                                               int nparts, long long n) {
  __shared__ float den;
  const int z = blockIdx.y;
  if (threadIdx.x == 0) {
    double t = 0;
    for (int k = 0; k < nparts; ++k) t += part[(long long)z * nparts + k];
    den = (float)(sqrt(t) + 1e-7);
  }
  __syncthreads();
  const float d = den;
  bf16* x = X + (long long)z * n;
  for (long long i = 4LL * ((long long)blockIdx.x * OPT_THREADS + threadIdx.x); i < n;
       i += 4LL * OPT_THREADS * gridDim.x) {
    bf16x4 v = *reinterpret_cast<const bf16x4*>(x + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (bf16)((float)v[e] / d);
    *reinterpret_cast<bf16x4*>(x + i) = v;
  }
}

// p -= step * X for matrix z = blockIdx.y; copy (may be null) receives the new weights in T.
template <typename T>
__global__ __launch_bounds__(OPT_THREADS) void muon_apply_kernel(float* __restrict__ p,
                                                                 T* __restrict__ copy,
                                                                 const bf16* __restrict__ X,
                                                                 MatGroup G, float step) {
  const int z = blockIdx.y;
  const long long n = (long long)G.rows * G.cols, off = mat_off(G, z);
  const bf16* x = X + (long long)z * n;
  for (long long i = 4LL * ((long long)blockIdx.x * OPT_THREADS + threadIdx.x); i < n;
       i += 4LL * OPT_THREADS * gridDim.x) {
    const bf16x4 xv = *reinterpret_cast<const bf16x4*>(x + i);
    f32x4 pv = *reinterpret_cast<const f32x4*>(p + off + i);
    float out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pv[e] -= step * (float)xv[e];
      out[e] = pv[e];
    }
    *reinterpret_cast<f32x4*>(p + off + i) = pv;
    if (copy) store4_opt(copy + off + i, out);
  }
}

// Partial sums per matrix in the momentum pass: about 64K elements each, at most 64.
int mom_parts(long long n) { return (int)std::max(1LL, std::min(64LL, n / 65536)); }

std::vector<MatGroup> muon_groups(const gpt_config& c, const Layout& L) {
  const long long D = c.d_model, F = c.d_mlp;
  const long long stride = c.n_layer > 1 ? L.wqkv[1] - L.wqkv[0] : 0;
  std::vector<MatGroup> g;
  g.push_back({L.wqkv[0], stride, D * D, 4, 4 * c.n_layer, (int)D, (int)D});  // q, k, v, o
  g.push_back({L.wfc[0], stride, 0, 1, c.n_layer, (int)F, (int)D});
  g.push_back({L.wpr[0], stride, 0, 1, c.n_layer, (int)D, (int)F});
  if (c.has_trigram) g.push_back({L.wtri, 0, 0, 1, 1, (int)D, (int)D});
  return g;
}

// Workspace: norm partials, the clip scalars, per-matrix partials, then X, X', A, B of the
// largest group (bf16).
struct OptWs {
  double *npart, *mpart;
  float* scal;
  bf16 *x0, *x1, *a, *b;
};
OptWs carve_opt(Carver& cv, const std::vector<MatGroup>& groups) {
  long long xmax = 0, smax = 0, pmax = 0;
  for (const MatGroup& G : groups) {
    const long long n = (long long)G.rows * G.cols, s = std::min(G.rows, G.cols);
    xmax = std::max(xmax, G.count * n);
    smax = std::max(smax, G.count * s * s);
    pmax = std::max(pmax, (long long)G.count * mom_parts(n));
  }
  OptWs w;
  w.npart = cv.take<double>(NORM_PARTS);
  w.scal = cv.take<float>(4);
  w.mpart = cv.take<double>(pmax);
  w.x0 = cv.take<bf16>(xmax);
  w.x1 = cv.take<bf16>(xmax);
  w.a = cv.take<bf16>(smax);
  w.b = cv.take<bf16>(smax);
  return w;
}

gpt_status check_groups(const gpt_config& c, const Layout& L) {
  const long long D = c.d_model;
  const long long stride = c.n_layer > 1 ? L.wqkv[1] - L.wqkv[0] : 0;
  for (int l = 0; l < c.n_layer; ++l)
    if (L.wqkv[l] != L.wqkv[0] + l * stride || L.wo[l] != L.wqkv[l] + 3 * D * D ||
        L.wfc[l] != L.wfc[0] + l * stride || L.wpr[l] != L.wpr[0] + l * stride)
      return fail(GPT_ESHAPE, "optimizer: unexpected parameter layout");
  return GPT_OK;
}

// Five (ns_steps) Newton-Schulz steps on the group's X (normalized, bf16) with three batched
// GEMMs each: A = X X^T (X^T X for tall matrices), B = c A A + b A, X' = B X + a X (X B + a X
// for tall matrices, B symmetric).  Returns the buffer holding the result.
gpt_status ns_iterate(const MatGroup& G, const OptWs& w, int steps, bf16** result, hipStream_t s) {
  const int R = G.rows, C = G.cols, Z = G.count;
  const bool tall = R > C;
  const int S = tall ? C : R;
  const long long xn = (long long)R * C, sn = (long long)S * S;
  bf16 *x = w.x0, *xn_ = w.x1;
  // the two symmetric products compute their upper-triangle tiles only when S is tile-aligned
  const bool sym = S % 256 == 0;
  auto gram = [&](auto epi) {
    return !tall ? gemm_batched<G_NS_GRAM>(true, true, S, S, C, x, C, xn, x, C, xn, Z, epi, s)
                 : gemm_batched<G_NS_GRAM>(false, false, S, S, R, x, C, xn, x, C, xn, Z, epi, s);
  };
  auto poly = [&](auto epi) {
    return gemm_batched<G_NS_POLY>(true, true, S, S, S, w.a, S, sn, w.a, S, sn, Z, epi, s);
  };
  for (int it = 0; it < steps; ++it) {
    gpt_status st = sym ? gram(EpiNsStoreSym{w.a, S, sn}) : gram(EpiNsStore{w.a, S, sn});
    if (st != GPT_OK) return st;
    st = sym ? poly(EpiNsCombineSym{w.b, w.a, S, sn, NS_C, NS_B})
             : poly(EpiNsCombine{w.b, w.a, S, sn, NS_C, NS_B});
    if (st != GPT_OK) return st;
    if (!tall)
      st = gemm_batched<G_NS_APPLY>(true, false, R, C, R, w.b, S, sn, x, C, xn, Z,
                                    EpiNsCombine{xn_, x, C, xn, 1.f, NS_A}, s);
    else
      st = gemm_batched<G_NS_APPLY>(true, true, R, C, C, x, C, xn, w.b, S, sn, Z,
                                    EpiNsCombine{xn_, x, C, xn, 1.f, NS_A}, s);
    if (st != GPT_OK) return st;
    std::swap(x, xn_);
  }
  *result = x;
  return GPT_OK;
}

unsigned grid_for(long long n, int per_block_elems) {
  return (unsigned)std::max(1LL, std::min(2048LL, (n + per_block_elems - 1) / per_block_elems));
}

template <typename T>
gpt_status opt_step(const gpt_config& c, const Layout& L, float* master, T* copy,
                    const float* grads, float* state, const gpt_opt_hparams& hp, const OptWs& w,
                    const std::vector<MatGroup>& groups, float* grad_norm, hipStream_t s) {
  const long long D = c.d_model, V = c.vocab, VD = V * D;
  const long long total = L.total;
  // 1. global norm and clip factor
  sumsq_kernel<<<NORM_PARTS, OPT_THREADS, 0, s>>>(grads, total, w.npart);
  clip_factor_kernel<<<1, NORM_PARTS, 0, s>>>(w.npart, hp.grad_clip, w.scal, grad_norm);
  // 2. Adam: token embedding and LM head (first moments in the momentum slots, second moments
  //    after the flat layout)
  const double scale = pow((double)D / 768.0, -0.5);
  const double bc1 = 1.0 - pow((double)hp.beta1, (double)hp.adam_step);
  const double bc2 = 1.0 - pow((double)hp.beta2, (double)hp.adam_step);
  float* v2 = state + total;
  struct AdamPart { long long off; float* v; double lr; };
  const AdamPart parts[2] = {{L.wte, v2, hp.lr_embedding * scale * hp.lr_mult},
                             {L.lm_head, v2 + align_elems(VD), hp.lr_unembedding * scale * hp.lr_mult}};
  for (const AdamPart& a : parts) {
    adam_kernel<T><<<grid_for(VD, OPT_THREADS * 4), OPT_THREADS, 0, s>>>(
        master + a.off, copy ? copy + a.off : nullptr, grads + a.off, state + a.off, a.v, VD,
        w.scal, (float)a.lr, hp.beta1, hp.beta2, (float)(a.lr / bc1), (float)(1.0 / sqrt(bc2)),
        hp.eps, hp.weight_decay);
  }
  // 3. Muon, one shape at a time
  for (const MatGroup& G : groups) {
    const long long n = (long long)G.rows * G.cols;
    const int np = mom_parts(n);
    muon_momentum_kernel<<<dim3(np, G.count), OPT_THREADS, 0, s>>>(
        grads, state, w.x0, w.mpart, G, w.scal, hp.momentum, hp.nesterov);
    ns_scale_kernel<<<dim3(grid_for(n, OPT_THREADS * 16), G.count), OPT_THREADS, 0, s>>>(
        w.x0, w.mpart, np, n);
    bf16* X = nullptr;
    gpt_status st = ns_iterate(G, w, hp.ns_steps, &X, s);
    if (st != GPT_OK) return st;
    const double step = hp.lr_matrix * hp.lr_mult * sqrt(std::max(1.0, (double)G.rows / G.cols));
    muon_apply_kernel<T><<<dim3(grid_for(n, OPT_THREADS * 16), G.count), OPT_THREADS, 0, s>>>(
        master, copy, X, G, (float)step);
  }
  return check_launch("optimizer step");
}

}  // namespace
}  // namespace gpt

using namespace gpt;

extern "C" {

int64_t gpt_opt_state_elems(const gpt_config* cfg) {
  if (validate(cfg) != GPT_OK) return -1;
  const Layout L = make_layout(*cfg);
  return L.total + 2 * align_elems((long long)cfg->vocab * cfg->d_model);
}

gpt_status gpt_opt_workspace_bytes(const gpt_config* cfg, size_t* bytes) {
  gpt_status st = validate(cfg);
  if (st != GPT_OK) return st;
  if (!bytes) return fail(GPT_EINVAL, "gpt_opt_workspace_bytes: bytes is null");
  const Layout L = make_layout(*cfg);
  Carver cv(nullptr, 0);
  carve_opt(cv, muon_groups(*cfg, L));
  *bytes = cv.size();
  return GPT_OK;
}

gpt_status gpt_opt_step(const gpt_config* cfg, float* master, void* params, const float* grads,
                        float* state, const gpt_opt_hparams* hp, void* workspace, size_t ws_bytes,
                        float* grad_norm, hipStream_t stream) {
  gpt_status st = validate(cfg);
  if (st != GPT_OK) return st;
  if (!hp || !master || !grads || !state) return fail(GPT_EINVAL, "gpt_opt_step: null argument");
  if (((uintptr_t)master | (uintptr_t)grads | (uintptr_t)state | (uintptr_t)params) % 16)
    return fail(GPT_EINVAL, "gpt_opt_step: buffers must be 16-byte aligned");
  if (hp->adam_step < 1 || hp->ns_steps < 0 || hp->ns_steps > 100 || !(hp->beta1 >= 0.f) ||
      !(hp->beta1 < 1.f) || !(hp->beta2 >= 0.f) || !(hp->beta2 < 1.f) || !(hp->eps >= 0.f) ||
      !(hp->momentum >= 0.f) || !(hp->momentum <= 1.f) || !(hp->grad_clip >= 0.f))
    return fail(GPT_ERANGE, "gpt_opt_step: hyperparameter out of range");
  const Layout L = make_layout(*cfg);
  if ((st = check_groups(*cfg, L)) != GPT_OK) return st;
  const std::vector<MatGroup> groups = muon_groups(*cfg, L);
  if (!workspace || (uintptr_t)workspace % 256)
    return fail(GPT_EINVAL, "gpt_opt_step: workspace must be non-null and 256-byte aligned");
  Carver cv(workspace, ws_bytes);
  const OptWs w = carve_opt(cv, groups);
  if (!cv.ok) return fail(GPT_EWORKSPACE, "gpt_opt_step: workspace too small");
  if (cfg->dtype == GPT_BF16)
    return opt_step<bf16>(*cfg, L, master, (bf16*)params, grads, state, *hp, w, groups, grad_norm,
                          stream);
  if (params && params != master)
    return fail(GPT_EINVAL, "gpt_opt_step: fp32 configurations update the master in place (params must be null or master)");
  return opt_step<float>(*cfg, L, master, nullptr, grads, state, *hp, w, groups, grad_norm, stream);
}

double gpt_lr_multiplier(int64_t it, int64_t num_iterations, double warmup_ratio,
                         double warmdown_ratio, double final_lr_frac) {
  const double warmup = nearbyint(warmup_ratio * (double)num_iterations);
  const double warmdown = nearbyint(warmdown_ratio * (double)num_iterations);
  if ((double)it < warmup) return ((double)it + 1.0) / warmup;
  if ((double)it <= (double)num_iterations - warmdown) return 1.0;
  const double progress = ((double)num_iterations - (double)it) / warmdown;
  return progress + (1.0 - progress) * final_lr_frac;
}

double gpt_muon_momentum(int64_t it) {
  const double frac = std::min((double)it / 300.0, 1.0);
  return (1.0 - frac) * 0.85 + frac * 0.95;
}

}  // extern "C"
