// Bandwidth-bound kernels of the step: rotary tables, embedding (+ its norm and the x0
// addend), weightless RMSNorm forward/backward, rotary + QK-norm forward/backward, and small
// elementwise helpers.  Definitions: the `norm`, `apply_rotary_emb` and
// `_precompute_rotary_embeddings` functions of the model posted in the "$1000 tier nanochat
// run" discussion; RMSNorm without affine parameters per the modded-nanogpt README.
//
// Row kernels use one 64-wide wavefront per row: each lane owns groups of 8 consecutive
// elements (16 B bf16 / 32 B fp32 vector accesses), the row statistic is a wave reduction,
// and nothing touches LDS.
#include "kernels.h"

namespace gpt {
namespace {

constexpr int ROWS_PER_BLOCK = 4;  // 4 waves of 64

// ------------------------------------------------------------------ rotary tables
// cos/sin [T, Hd/2] of t * base^(-2i/Hd), computed in double, stored rounded to T.
template <typename T>
__global__ void rope_table_kernel(T* cos_t, T* sin_t, int Tn, int half, int hd, double base) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= Tn * half) return;
  const int t = idx / half, i = idx % half;
  const double inv = pow(base, -(2.0 * i) / (double)hd);
  const double a = (double)t * inv;
  cos_t[idx] = from_f32<T>((float)cos(a));
  sin_t[idx] = from_f32<T>((float)sin(a));
}

// ------------------------------------------------------------------ embedding
// x[t] = rms(wte[tok[t]]) + x0_add[t]  (fp32 out); rstd[t]; clamped token ids to tok_c.
template <typename T, int MAXG>
__global__ __launch_bounds__(256) void embed_fwd_kernel(
    const int32_t* __restrict__ tok, const T* __restrict__ wte, const T* __restrict__ x0_add,
    float* __restrict__ x, float* __restrict__ rstd, int32_t* __restrict__ tok_c, int* err,
    long long N, int D, int V, float eps) {
  const long long row = (long long)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / WAVE;
  if (row >= N) return;
  const int lane = threadIdx.x % WAVE, groups = D / 8;
  int id = tok[row];
  if (id < 0 || id >= V) {
    if (lane == 0) atomicOr(err, 1);
    id = id < 0 ? 0 : V - 1;
  }
  if (lane == 0) tok_c[row] = id;
  float v[MAXG][8];
  float ss = 0.f;
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi) {
    const int g = lane + gi * WAVE;
    if (g < groups) {
      load8_f32(wte + (size_t)id * D + g * 8, v[gi]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[gi][e] * v[gi][e];
    }
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)D + eps);
  if (lane == 0) rstd[row] = r;
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi) {
    const int g = lane + gi * WAVE;
    if (g < groups) {
      float a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (x0_add) load8_f32(x0_add + row * D + g * 8, a);
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = v[gi][e] * r + a[e];
      store8_f32(x + row * D + g * 8, o);
    }
  }
}

// de[t] = rms_bwd(e = wte[tok_c[t]], r[t], dx[t]) (fp32).
template <typename T, int MAXG>
__global__ __launch_bounds__(256) void embed_bwd_kernel(
    const int32_t* __restrict__ tok_c, const T* __restrict__ wte, const float* __restrict__ rstd,
    const float* __restrict__ dx, float* __restrict__ de, long long N, int D) {
  const long long row = (long long)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / WAVE;
  if (row >= N) return;
  const int lane = threadIdx.x % WAVE, groups = D / 8;
  const int id = tok_c[row];
  const float r = rstd[row];
  float y[MAXG][8], g_[MAXG][8];
  float dot = 0.f;
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi) {
    const int g = lane + gi * WAVE;
    if (g < groups) {
      load8_f32(wte + (size_t)id * D + g * 8, y[gi]);
      load8_f32(dx + row * D + g * 8, g_[gi]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[gi][e] *= r;
        dot += y[gi][e] * g_[gi][e];
      }
    }
  }
  const float mean = wave_sum(dot) / (float)D;
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi) {
    const int g = lane + gi * WAVE;
    if (g < groups) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = r * (g_[gi][e] - y[gi][e] * mean);
      store8_f32(de + row * D + g * 8, o);
    }
  }
}

// ------------------------------------------------------------------ RMSNorm
// y = x * r, r = 1/sqrt(mean(x^2) + eps); x fp32 -> y in T.
template <typename T, int MAXG>
__global__ __launch_bounds__(256) void rms_fwd_kernel(const float* __restrict__ x,
                                                      T* __restrict__ y, float* __restrict__ rstd,
                                                      long long N, int D, float eps) {
  const long long row = (long long)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / WAVE;
  if (row >= N) return;
  const int lane = threadIdx.x % WAVE, groups = D / 8;
  float v[MAXG][8];
  float ss = 0.f;
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi) {
    const int g = lane + gi * WAVE;
    if (g < groups) {
      load8_f32(x + row * D + g * 8, v[gi]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += v[gi][e] * v[gi][e];
    }
  }
  ss = wave_sum(ss);
  const float r = 1.f / sqrtf(ss / (float)D + eps);
  if (lane == 0) rstd[row] = r;
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi) {
    const int g = lane + gi * WAVE;
    if (g < groups) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = v[gi][e] * r;
      store8_f32(y + row * D + g * 8, o);
    }
  }
}

// dx = dres + r * (dy - y * mean(dy * y)),  y = x * r.  dres may alias dx.  dx_t (optional)
// receives dx rounded to T (the operand of the next weight-gradient GEMM).
template <typename T, int MAXG>
__global__ __launch_bounds__(256) void rms_bwd_kernel(
    const float* __restrict__ x, const float* __restrict__ rstd, const float* __restrict__ dy,
    const float* dres, float* dx, T* __restrict__ dx_t, long long N, int D) {
  const long long row = (long long)blockIdx.x * ROWS_PER_BLOCK + threadIdx.x / WAVE;
  if (row >= N) return;
  const int lane = threadIdx.x % WAVE, groups = D / 8;
  const float r = rstd[row];
  float y[MAXG][8], g_[MAXG][8];
  float dot = 0.f;
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi) {
    const int g = lane + gi * WAVE;
    if (g < groups) {
      load8_f32(x + row * D + g * 8, y[gi]);
      load8_f32(dy + row * D + g * 8, g_[gi]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[gi][e] *= r;
        dot += y[gi][e] * g_[gi][e];
      }
    }
  }
  const float mean = wave_sum(dot) / (float)D;
#pragma unroll
  for (int gi = 0; gi < MAXG; ++gi) {
    const int g = lane + gi * WAVE;
    if (g < groups) {
      float o[8];
      if (dres) {
        load8_f32(dres + row * D + g * 8, o);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += r * (g_[gi][e] - y[gi][e] * mean);
      store8_f32(dx + row * D + g * 8, o);
      if (dx_t) store8_f32(dx_t + row * D + g * 8, o);
    }
  }
}

// ------------------------------------------------------------------ rotary + QK-norm
// In place on the q and k column blocks of qkv [N, 3D].  One thread per 8 consecutive rotation
// pairs (i..i+7, i+half..i+half+7) of one head: 16-byte (bf16) / 32-byte (fp32) accesses; the
// Hd/16 lanes of a head reduce the head's sum of squares.  rstd_qk [N, 2H]: q heads then k heads.
template <typename T>
__global__ __launch_bounds__(256) void rope_qknorm_fwd_kernel(
    T* __restrict__ qkv, const T* __restrict__ cos_t, const T* __restrict__ sin_t,
    float* __restrict__ rstd_qk, long long N, int Tn, int H, int hd, int qk_norm, float eps) {
  const int D = H * hd, half = hd / 2, per_tok = D / 8;  // threads per token (q and k)
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= N * per_tok) return;  // per_tok is a multiple of hd/16: whole lane groups exit together
  const long long tok = gid / per_tok;
  const int p = (int)(gid % per_tok) * 8;
  const int hq = p / half, i = p % half;
  const int t = (int)(tok % Tn);
  T* base = qkv + tok * 3 * D + (hq < H ? 0 : D) + (hq % H) * hd;
  float x1[8], x2[8], c[8], sn[8], y1[8], y2[8];
  load8_f32(base + i, x1);
  load8_f32(base + i + half, x2);
  load8_f32(cos_t + t * half + i, c);
  load8_f32(sin_t + t * half + i, sn);
  float ss = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    y1[e] = x1[e] * c[e] + x2[e] * sn[e];
    y2[e] = -x1[e] * sn[e] + x2[e] * c[e];
    ss += y1[e] * y1[e] + y2[e] * y2[e];
  }
  float r = 1.f;
  if (qk_norm) {
    ss = group_sum(ss, half / 8);
    r = 1.f / sqrtf(ss / (float)hd + eps);
    if (i == 0) rstd_qk[tok * 2 * H + hq] = r;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    y1[e] *= r;
    y2[e] *= r;
  }
  store8_f32(base + i, y1);
  store8_f32(base + i + half, y2);
}

// Backward on the dq, dk column blocks of dqkv, in place: dz = r (dy - y mean(dy y)) with y
// the saved normalized q/k, then the transposed rotation dx1 = dz1 c - dz2 s,
// dx2 = dz1 s + dz2 c.
template <typename T>
__global__ __launch_bounds__(256) void rope_qknorm_bwd_kernel(
    T* __restrict__ dqkv, const T* __restrict__ qkv, const T* __restrict__ cos_t,
    const T* __restrict__ sin_t, const float* __restrict__ rstd_qk, long long N, int Tn, int H,
    int hd, int qk_norm) {
  const int D = H * hd, half = hd / 2, per_tok = D / 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= N * per_tok) return;
  const long long tok = gid / per_tok;
  const int p = (int)(gid % per_tok) * 8;
  const int hq = p / half, i = p % half;
  const int t = (int)(tok % Tn);
  const long long off = tok * 3 * D + (hq < H ? 0 : D) + (hq % H) * hd;
  float d1[8], d2[8], c[8], sn[8], o1[8], o2[8];
  load8_f32(dqkv + off + i, d1);
  load8_f32(dqkv + off + i + half, d2);
  if (qk_norm) {
    float y1[8], y2[8];
    load8_f32(qkv + off + i, y1);
    load8_f32(qkv + off + i + half, y2);
    const float r = rstd_qk[tok * 2 * H + hq];
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += d1[e] * y1[e] + d2[e] * y2[e];
    const float mean = group_sum(dot, half / 8) / (float)hd;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      d1[e] = r * (d1[e] - y1[e] * mean);
      d2[e] = r * (d2[e] - y2[e] * mean);
    }
  }
  load8_f32(cos_t + t * half + i, c);
  load8_f32(sin_t + t * half + i, sn);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    o1[e] = d1[e] * c[e] - d2[e] * sn[e];
    o2[e] = d1[e] * sn[e] + d2[e] * c[e];
  }
  store8_f32(dqkv + off + i, o1);
  store8_f32(dqkv + off + i + half, o2);
}

// ------------------------------------------------------------------ workspace guards
// Guard g of the table covers bytes [tab[g], tab[g] + GUARD_BYTES) of the workspace; one
// workgroup per guard, one 32-bit word per thread.
__global__ void guard_fill_kernel(char* __restrict__ ws, const long long* __restrict__ tab) {
  uint32_t* w = reinterpret_cast<uint32_t*>(ws + tab[blockIdx.x]);
  w[threadIdx.x] = GUARD_WORD;
}
__global__ void guard_check_kernel(const char* __restrict__ ws, const long long* __restrict__ tab,
                                   int* __restrict__ err) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(ws + tab[blockIdx.x]);
  if (w[threadIdx.x] != GUARD_WORD) atomicOr(err, 4);
}

// ------------------------------------------------------------------ elementwise helpers
__global__ void fill_f32_kernel(float* p, long long n, float v) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// dst[r, :] (+)= src[r*lds + :] for rows of width D (8-element vectors); dst fp32.
template <typename T>
__global__ void accum_rows_kernel(float* __restrict__ dst, const T* __restrict__ src,
                                  long long lds, long long N, int D, int add) {
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int groups = D / 8;
  if (gid >= N * groups) return;
  const long long r = gid / groups;
  const int g = (int)(gid % groups);
  float a[8], b[8];
  load8_f32(src + r * lds + g * 8, b);
  if (add) {
    load8_f32(dst + r * D + g * 8, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] += a[e];
  }
  store8_f32(dst + r * D + g * 8, b);
}

// dst (T) = src (fp32), n a multiple of 8.
template <typename T>
__global__ void cast_kernel(T* __restrict__ dst, const float* __restrict__ src, long long n8) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n8) return;
  float v[8];
  load8_f32(src + i * 8, v);
  store8_f32(dst + i * 8, v);
}

template <int MAXG_, typename F>
gpt_status dispatch_width(int D, F&& f) {
  const int maxg = (D / 8 + WAVE - 1) / WAVE;
  switch (maxg) {
    case 1: f(std::integral_constant<int, 1>()); break;
    case 2: f(std::integral_constant<int, 2>()); break;
    case 3: f(std::integral_constant<int, 3>()); break;
    case 4: f(std::integral_constant<int, 4>()); break;
    default: return fail(GPT_ESHAPE, "row width above 2048 is not supported");
  }
  return GPT_OK;
}

}  // namespace

template <typename T>
gpt_status launch_rope_table(T* cos_t, T* sin_t, int Tn, int hd, float base, hipStream_t s) {
  const int half = hd / 2;
  rope_table_kernel<T><<<cdiv((long long)Tn * half, 256), 256, 0, s>>>(cos_t, sin_t, Tn, half, hd,
                                                                       (double)base);
  return check_launch("rope table");
}

template <typename T>
gpt_status launch_embed_fwd(const int32_t* tok, const T* wte, const T* x0_add, float* x,
                            float* rstd, int32_t* tok_c, int* err, long long N, int D, int V,
                            float eps, hipStream_t s) {
  gpt_status st = dispatch_width<4>(D, [&](auto G) {
    embed_fwd_kernel<T, decltype(G)::value><<<cdiv(N, ROWS_PER_BLOCK), 256, 0, s>>>(
        tok, wte, x0_add, x, rstd, tok_c, err, N, D, V, eps);
  });
  return st != GPT_OK ? st : check_launch("embed fwd");
}

template <typename T>
gpt_status launch_embed_bwd(const int32_t* tok_c, const T* wte, const float* rstd,
                            const float* dx, float* de, long long N, int D, hipStream_t s) {
  gpt_status st = dispatch_width<4>(D, [&](auto G) {
    embed_bwd_kernel<T, decltype(G)::value><<<cdiv(N, ROWS_PER_BLOCK), 256, 0, s>>>(
        tok_c, wte, rstd, dx, de, N, D);
  });
  return st != GPT_OK ? st : check_launch("embed bwd");
}

template <typename T>
gpt_status launch_rms_fwd(const float* x, T* y, float* rstd, long long N, int D, float eps,
                          hipStream_t s) {
  gpt_status st = dispatch_width<4>(D, [&](auto G) {
    rms_fwd_kernel<T, decltype(G)::value><<<cdiv(N, ROWS_PER_BLOCK), 256, 0, s>>>(x, y, rstd, N,
                                                                                  D, eps);
  });
  return st != GPT_OK ? st : check_launch("rmsnorm fwd");
}

template <typename T>
gpt_status launch_rms_bwd(const float* x, const float* rstd, const float* dy, const float* dres,
                          float* dx, T* dx_t, long long N, int D, hipStream_t s) {
  gpt_status st = dispatch_width<4>(D, [&](auto G) {
    rms_bwd_kernel<T, decltype(G)::value><<<cdiv(N, ROWS_PER_BLOCK), 256, 0, s>>>(
        x, rstd, dy, dres, dx, dx_t, N, D);
  });
  return st != GPT_OK ? st : check_launch("rmsnorm bwd");
}

template <typename T>
gpt_status launch_rope_qknorm_fwd(T* qkv, const T* cos_t, const T* sin_t, float* rstd_qk,
                                  long long N, int Tn, int H, int hd, int qk_norm, float eps,
                                  hipStream_t s) {
  rope_qknorm_fwd_kernel<T><<<cdiv(N * H * hd / 8, 256), 256, 0, s>>>(qkv, cos_t, sin_t, rstd_qk,
                                                                      N, Tn, H, hd, qk_norm, eps);
  return check_launch("rope+qknorm fwd");
}

template <typename T>
gpt_status launch_rope_qknorm_bwd(T* dqkv, const T* qkv, const T* cos_t, const T* sin_t,
                                  const float* rstd_qk, long long N, int Tn, int H, int hd,
                                  int qk_norm, hipStream_t s) {
  rope_qknorm_bwd_kernel<T><<<cdiv(N * H * hd / 8, 256), 256, 0, s>>>(dqkv, qkv, cos_t, sin_t,
                                                                      rstd_qk, N, Tn, H, hd, qk_norm);
  return check_launch("rope+qknorm bwd");
}

gpt_status launch_guards(char* ws, const long long* tab, int n, int* err, int check,
                         hipStream_t s) {
  if (n == 0) return GPT_OK;
  constexpr int W = (int)(GUARD_BYTES / 4);
  if (check) guard_check_kernel<<<n, W, 0, s>>>(ws, tab, err);
  else guard_fill_kernel<<<n, W, 0, s>>>(ws, tab);
  return check_launch("workspace guards");
}

gpt_status launch_fill(float* p, long long n, float v, hipStream_t s) {
  if (n == 0) return GPT_OK;
  fill_f32_kernel<<<cdiv(n, 256), 256, 0, s>>>(p, n, v);
  return check_launch("fill");
}

template <typename T>
gpt_status launch_accum_rows(float* dst, const T* src, long long lds, long long N, int D, int add,
                             hipStream_t s) {
  accum_rows_kernel<T><<<cdiv(N * (D / 8), 256), 256, 0, s>>>(dst, src, lds, N, D, add);
  return check_launch("accumulate rows");
}

template <typename T>
gpt_status launch_cast(T* dst, const float* src, long long n, hipStream_t s) {
  cast_kernel<T><<<cdiv(n / 8, 256), 256, 0, s>>>(dst, src, n / 8);
  return check_launch("cast");
}

#define INST(T)                                                                                  \
  template gpt_status launch_rope_table<T>(T*, T*, int, int, float, hipStream_t);               \
  template gpt_status launch_embed_fwd<T>(const int32_t*, const T*, const T*, float*, float*,   \
                                          int32_t*, int*, long long, int, int, float,           \
                                          hipStream_t);                                          \
  template gpt_status launch_embed_bwd<T>(const int32_t*, const T*, const float*, const float*, \
                                          float*, long long, int, hipStream_t);                 \
  template gpt_status launch_rms_fwd<T>(const float*, T*, float*, long long, int, float,        \
                                        hipStream_t);                                            \
  template gpt_status launch_rms_bwd<T>(const float*, const float*, const float*, const float*, \
                                        float*, T*, long long, int, hipStream_t);               \
  template gpt_status launch_rope_qknorm_fwd<T>(T*, const T*, const T*, float*, long long, int,  \
                                                int, int, int, float, hipStream_t);             \
  template gpt_status launch_rope_qknorm_bwd<T>(T*, const T*, const T*, const T*, const float*, \
                                                long long, int, int, int, int, hipStream_t);    \
  template gpt_status launch_accum_rows<T>(float*, const T*, long long, long long, int, int,     \
                                           hipStream_t);                                         \
  template gpt_status launch_cast<T>(T*, const float*, long long, hipStream_t);
INST(float)
INST(bf16)
#undef INST

}  // namespace gpt
