// Causal flash attention forward and backward on gfx950 matrix cores.
//
// Definition (CausalSelfAttention.forward in the "$1000 tier nanochat run" discussion):
// O = softmax(q k^T / sqrt(Hd) with keys s <= t) v, per batch row and head; q and k have been
// rotated and RMS-normalised.  Backward: dV = P^T dO, dP = dO V^T,
// dS = P (dP - rowsum(dO * O)), dQ = dS K / sqrt(Hd), dK = dS^T Q / sqrt(Hd).
//
// Layout: q, k, v live in one [N, 3D] buffer (token-major, head h at columns h*Hd of each
// block); O is [N, D]; the forward saves the base-2 log-sum-exp LSE2 [B, H, T] of the scaled
// scores.  MFMA is v_mfma_f32_32x32x16_bf16 (fp32: 8 x v_mfma_f32_32x32x2f32), whose output
// tile holds, in lane l and register r, row (r/4)*8 + (l/32)*4 + r%4 and column l%32.
//
//  * forward and dQ put queries on lanes: S^T = K Q^T, so every softmax row sits in one lane
//    pair (l, l^32) and needs a single cross-lane exchange;
//  * dK/dV puts keys on lanes: S = Q K^T, dV^T = dO^T P, dK^T = Q^T dS;
//  * an accumulator's registers 8h..8h+7 are used directly as the 16-wide K operand of the
//    next MFMA; the other operand is read from an LDS tile stored transposed, with the same
//    permutation of the 16 K positions (rows g*4..g*4+3 and 8+g*4..8+g*4+3 for lane group g);
//  * causal work is skipped per 32-row wave, and the heaviest blocks launch first.
// No atomics: dQ comes from its own kernel, so results are bitwise reproducible.
#include "kernels.h"

namespace gpt {
namespace {

constexpr int ATHREADS = 256;  // 4 waves

template <typename T> struct Vec4;
template <> struct Vec4<bf16> { typedef bf16x4 type; };
template <> struct Vec4<float> { typedef f32x4 type; };
template <typename T> using vec4_t = typename Vec4<T>::type;

template <typename T> struct MmaA;
template <> struct MmaA<bf16> {
  static __device__ __forceinline__ void run(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
};
template <> struct MmaA<float> {
  static __device__ __forceinline__ void run(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
  }
};
template <typename T>
__device__ __forceinline__ void mma(f32x16& acc, const vec8_t<T>& a, const vec8_t<T>& b) {
  MmaA<T>::run(acc, a, b);
}

template <typename T> constexpr int pad() { return 16 / sizeof(T); }

// 8 consecutive elements [row][k0 + g*8 ..]
template <typename T>
__device__ __forceinline__ vec8_t<T> frag_rows(const T* lds, int pitch, int row, int k0, int g) {
  return load8(lds + row * pitch + k0 + g * 8);
}
// K positions permuted like accumulator registers: [row][k0+g*4 ..+3] and [row][k0+8+g*4 ..+3]
template <typename T>
__device__ __forceinline__ vec8_t<T> frag_split(const T* lds, int pitch, int row, int k0, int g) {
  const vec4_t<T> a = *reinterpret_cast<const vec4_t<T>*>(lds + row * pitch + k0 + g * 4);
  const vec4_t<T> b = *reinterpret_cast<const vec4_t<T>*>(lds + row * pitch + k0 + 8 + g * 4);
  vec8_t<T> v;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
  return v;
}
template <typename T>
__device__ __forceinline__ vec8_t<T> acc_frag(const f32x16& acc, int h) {
  vec8_t<T> v;
#pragma unroll
  for (int s = 0; s < 8; ++s) v[s] = from_f32<T>(acc[h * 8 + s]);
  return v;
}

// Rows [r0, r0+R) x HD columns of a matrix with row stride ld -> lds[r][d] (rows >= lim: 0).
template <typename T, int R, int HD>
__device__ __forceinline__ void stage_rows(T* lds, int pitch, const T* __restrict__ g,
                                           long long ld, int r0, int lim) {
  constexpr int NV = R * HD / 8;
  for (int v = threadIdx.x; v < NV; v += ATHREADS) {
    const int r = v / (HD / 8), c = (v % (HD / 8)) * 8;
    vec8_t<T> x = (r0 + r < lim) ? load8(g + (long long)(r0 + r) * ld + c) : vec8_t<T>{};
    store8(lds + r * pitch + c, x);
  }
}
// Same rows, transposed: lds[d][r].
template <typename T, int R, int HD>
__device__ __forceinline__ void stage_transposed(T* lds, int pitch, const T* __restrict__ g,
                                                 long long ld, int r0, int lim) {
  constexpr int NB = (R / 8) * (HD / 8);
  for (int b = threadIdx.x; b < NB; b += ATHREADS) {
    const int rb = b % (R / 8), db = b / (R / 8);
    vec8_t<T> in[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int r = r0 + rb * 8 + k;
      in[k] = (r < lim) ? load8(g + (long long)r * ld + db * 8) : vec8_t<T>{};
    }
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      vec8_t<T> o;
#pragma unroll
      for (int k = 0; k < 8; ++k) o[k] = in[k][d];
      store8(lds + (db * 8 + d) * pitch + rb * 8, o);
    }
  }
}

// Output of a [HD x 32] transposed accumulator set (lane = row l%32 of the result) stored as
// rows of a token-major matrix: element (row, d) with d = dt*32 + (r/4)*8 + g*4 + r%4.
template <typename T, int HD>
__device__ __forceinline__ void store_acc_rows(T* __restrict__ dst_row, const f32x16 (&acc)[HD / 32],
                                               float scale, int g) {
#pragma unroll
  for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      vec4_t<T> v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = from_f32<T>(acc[dt][q * 4 + i] * scale);
      *reinterpret_cast<vec4_t<T>*>(dst_row + dt * 32 + q * 8 + g * 4) = v;
    }
}

// ------------------------------------------------------------------ forward
template <typename T, int HD>
__global__ __launch_bounds__(ATHREADS, 2) void attn_fwd_kernel(const T* __restrict__ qkv,
                                                               T* __restrict__ out,
                                                               float* __restrict__ lse2,
                                                               int Tn, int H, float sl2) {
  constexpr int BKV = 64, PK = HD + pad<T>(), PV = BKV + pad<T>();
  __shared__ __attribute__((aligned(16))) T Ks[BKV * PK];
  __shared__ __attribute__((aligned(16))) T Vt[HD * PV];
  const int D = H * HD;
  const long long ld = 3LL * D;
  const int qb = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE, lr = lane % 32, g = lane / 32;
  const int q0 = qb * 128 + w * 32, q = q0 + lr;
  const bool active = q0 < Tn;
  const T* base = qkv + (long long)b * Tn * ld;

  vec8_t<T> qf[HD / 16];
  if (active) {
#pragma unroll
    for (int c = 0; c < HD / 16; ++c) qf[c] = load8(base + (long long)q * ld + h * HD + c * 16 + g * 8);
  }
  f32x16 o[HD / 32];
#pragma unroll
  for (int i = 0; i < HD / 32; ++i) o[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  const int kv_end = min(Tn, (qb + 1) * 128);
  for (int kv0 = 0; kv0 < kv_end; kv0 += BKV) {
    __syncthreads();
    stage_rows<T, BKV, HD>(Ks, PK, base + D + h * HD, ld, kv0, Tn);
    stage_transposed<T, BKV, HD>(Vt, PV, base + 2 * D + h * HD, ld, kv0, Tn);
    __syncthreads();
    if (!active || kv0 > q0 + 31) continue;
    f32x16 s[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      s[st] = f32x16{};
#pragma unroll
      for (int c = 0; c < HD / 16; ++c) mma<T>(s[st], frag_rows(Ks, PK, st * 32 + lr, c * 16, g), qf[c]);
    }
    const bool diag = kv0 + BKV - 1 > q0;
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float v = s[st][r] * sl2;
        if (diag) {
          const int key = kv0 + st * 32 + (r / 4) * 8 + g * 4 + (r % 4);
          if (key > q) v = -INFINITY;
        }
        s[st][r] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float mn = fmaxf(m, mx);
    const float alpha = exp2f(m - mn);
    float sum = 0.f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = exp2f(s[st][r] - mn);
        s[st][r] = p;
        sum += p;
      }
    sum += __shfl_xor(sum, 32, WAVE);
    l = l * alpha + sum;
    m = mn;
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    vec8_t<T> pf[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) pf[st][hh] = acc_frag<T>(s[st], hh);
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          mma<T>(o[dt], frag_split(Vt, PV, dt * 32 + lr, st * 32 + hh * 16, g), pf[st][hh]);
  }
  if (!active) return;
  T* dst = out + ((long long)b * Tn + q) * D + h * HD;
  store_acc_rows<T, HD>(dst, o, 1.f / l, g);
  if (g == 0) lse2[((long long)b * H + h) * Tn + q] = m + log2f(l);
}

// ------------------------------------------------------------------ backward
// Dq[b,h,t] = sum_d dO[t,d] * O[t,d]
template <typename T, int HD>
__global__ void attn_bwd_pre_kernel(const T* __restrict__ o, const T* __restrict__ dout,
                                    float* __restrict__ dq_sum, long long N, int Tn, int H) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * H) return;
  const long long tok = i / H;
  const int h = (int)(i % H);
  const int D = H * HD;
  const T* a = o + tok * D + h * HD;
  const T* d = dout + tok * D + h * HD;
  float s = 0.f;
#pragma unroll 2
  for (int c = 0; c < HD; c += 8) {
    float x[8], y[8];
    load8_f32(a + c, x);
    load8_f32(d + c, y);
#pragma unroll
    for (int e = 0; e < 8; ++e) s += x[e] * y[e];
  }
  const long long b = tok / Tn, t = tok % Tn;
  dq_sum[(b * H + h) * Tn + t] = s;
}

// dK, dV for 128 keys per workgroup (4 waves x 32 keys), looping over 32-query tiles.
template <typename T, int HD>
__global__ __launch_bounds__(ATHREADS, HD >= 128 ? 1 : 2) void attn_bwd_dkdv_kernel(
    const T* __restrict__ qkv, const T* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ dq_sum, T* __restrict__ dqkv, int Tn, int H, float sl2,
    float scale) {
  constexpr int BQ = 32, PR = HD + pad<T>(), PT = BQ + pad<T>();
  __shared__ __attribute__((aligned(16))) T Qs[BQ * PR];
  __shared__ __attribute__((aligned(16))) T Qt[HD * PT];
  __shared__ __attribute__((aligned(16))) T Os[BQ * PR];
  __shared__ __attribute__((aligned(16))) T Ot[HD * PT];
  __shared__ float lse_s[BQ], dsum_s[BQ];
  const int D = H * HD;
  const long long ld = 3LL * D;
  const int kb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;  // key block 0 is the heaviest
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE, lr = lane % 32, g = lane / 32;
  const int k0 = kb * 128 + w * 32, key = k0 + lr;
  const bool active = k0 < Tn;
  const T* base = qkv + (long long)b * Tn * ld;
  const T* dbase = dout + (long long)b * Tn * D;
  const float* lrow = lse2 + ((long long)b * H + h) * Tn;
  const float* drow = dq_sum + ((long long)b * H + h) * Tn;

  vec8_t<T> kf[HD / 16], vf[HD / 16];
  if (active) {
#pragma unroll
    for (int c = 0; c < HD / 16; ++c) {
      kf[c] = load8(base + (long long)key * ld + D + h * HD + c * 16 + g * 8);
      vf[c] = load8(base + (long long)key * ld + 2 * D + h * HD + c * 16 + g * 8);
    }
  }
  f32x16 dk[HD / 32], dv[HD / 32];
#pragma unroll
  for (int i = 0; i < HD / 32; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  for (int q0 = kb * 128; q0 < Tn; q0 += BQ) {
    __syncthreads();
    stage_rows<T, BQ, HD>(Qs, PR, base + h * HD, ld, q0, Tn);
    stage_transposed<T, BQ, HD>(Qt, PT, base + h * HD, ld, q0, Tn);
    stage_rows<T, BQ, HD>(Os, PR, dbase + h * HD, D, q0, Tn);
    stage_transposed<T, BQ, HD>(Ot, PT, dbase + h * HD, D, q0, Tn);
    if (threadIdx.x < BQ) {
      lse_s[threadIdx.x] = lrow[q0 + threadIdx.x];
      dsum_s[threadIdx.x] = drow[q0 + threadIdx.x];
    }
    __syncthreads();
    if (!active || q0 + BQ - 1 < k0) continue;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int c = 0; c < HD / 16; ++c) {
      mma<T>(s, frag_rows(Qs, PR, lr, c * 16, g), kf[c]);
      mma<T>(dp, frag_rows(Os, PR, lr, c * 16, g), vf[c]);
    }
    const bool diag = q0 < k0 + 31;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qi = (r / 4) * 8 + g * 4 + (r % 4);
      float p = exp2f(s[r] * sl2 - lse_s[qi]);
      if (diag && key > q0 + qi) p = 0.f;
      s[r] = p;
      dp[r] = p * (dp[r] - dsum_s[qi]);
    }
    vec8_t<T> pf[2], sf[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      pf[hh] = acc_frag<T>(s, hh);
      sf[hh] = acc_frag<T>(dp, hh);
    }
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        mma<T>(dv[dt], frag_split(Ot, PT, dt * 32 + lr, hh * 16, g), pf[hh]);
        mma<T>(dk[dt], frag_split(Qt, PT, dt * 32 + lr, hh * 16, g), sf[hh]);
      }
  }
  if (!active) return;
  T* row = dqkv + ((long long)b * Tn + key) * ld + h * HD;
  store_acc_rows<T, HD>(row + D, dk, scale, g);
  store_acc_rows<T, HD>(row + 2 * D, dv, 1.f, g);
}

// dQ for 128 queries per workgroup, looping over 64-key tiles.
template <typename T, int HD>
__global__ __launch_bounds__(ATHREADS, 2) void attn_bwd_dq_kernel(
    const T* __restrict__ qkv, const T* __restrict__ dout, const float* __restrict__ lse2,
    const float* __restrict__ dq_sum, T* __restrict__ dqkv, int Tn, int H, float sl2,
    float scale) {
  constexpr int BKV = 64, PR = HD + pad<T>(), PT = BKV + pad<T>();
  __shared__ __attribute__((aligned(16))) T Ks[BKV * PR];
  __shared__ __attribute__((aligned(16))) T Vs[BKV * PR];
  __shared__ __attribute__((aligned(16))) T Kt[HD * PT];
  const int D = H * HD;
  const long long ld = 3LL * D;
  const int qb = gridDim.x - 1 - blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE, lr = lane % 32, g = lane / 32;
  const int q0 = qb * 128 + w * 32, q = q0 + lr;
  const bool active = q0 < Tn;
  const T* base = qkv + (long long)b * Tn * ld;
  vec8_t<T> qf[HD / 16], of[HD / 16];
  float lq = 0.f, dsum = 0.f;
  if (active) {
#pragma unroll
    for (int c = 0; c < HD / 16; ++c) {
      qf[c] = load8(base + (long long)q * ld + h * HD + c * 16 + g * 8);
      of[c] = load8(dout + ((long long)b * Tn + q) * D + h * HD + c * 16 + g * 8);
    }
    lq = lse2[((long long)b * H + h) * Tn + q];
    dsum = dq_sum[((long long)b * H + h) * Tn + q];
  }
  f32x16 dq[HD / 32];
#pragma unroll
  for (int i = 0; i < HD / 32; ++i) dq[i] = f32x16{};
  const int kv_end = min(Tn, (qb + 1) * 128);
  for (int kv0 = 0; kv0 < kv_end; kv0 += BKV) {
    __syncthreads();
    stage_rows<T, BKV, HD>(Ks, PR, base + D + h * HD, ld, kv0, Tn);
    stage_rows<T, BKV, HD>(Vs, PR, base + 2 * D + h * HD, ld, kv0, Tn);
    stage_transposed<T, BKV, HD>(Kt, PT, base + D + h * HD, ld, kv0, Tn);
    __syncthreads();
    if (!active || kv0 > q0 + 31) continue;
    const bool diag = kv0 + BKV - 1 > q0;
    vec8_t<T> sf[2][2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < HD / 16; ++c) {
        mma<T>(s, frag_rows(Ks, PR, st * 32 + lr, c * 16, g), qf[c]);
        mma<T>(dp, frag_rows(Vs, PR, st * 32 + lr, c * 16, g), of[c]);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kv0 + st * 32 + (r / 4) * 8 + g * 4 + (r % 4);
        float p = exp2f(s[r] * sl2 - lq);
        if (diag && key > q) p = 0.f;
        dp[r] = p * (dp[r] - dsum);
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) sf[st][hh] = acc_frag<T>(dp, hh);
    }
#pragma unroll
    for (int dt = 0; dt < HD / 32; ++dt)
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
          mma<T>(dq[dt], frag_split(Kt, PT, dt * 32 + lr, st * 32 + hh * 16, g), sf[st][hh]);
  }
  if (!active) return;
  store_acc_rows<T, HD>(dqkv + ((long long)b * Tn + q) * ld + h * HD, dq, scale, g);
}

// bf16: head_dim 32, 64, 128; fp32: 32, 64 (the fp32 path exists for small parity configs).
template <typename T, typename F>
gpt_status dispatch_hd(int hd, F&& f) {
  switch (hd) {
    case 32: f(std::integral_constant<int, 32>()); break;
    case 64: f(std::integral_constant<int, 64>()); break;
    case 128:
      if constexpr (std::is_same<T, bf16>::value) {
        f(std::integral_constant<int, 128>());
        break;
      }
      [[fallthrough]];
    default: return fail(GPT_ESHAPE, "attention head_dim must be 32, 64 or 128 (fp32: 32 or 64)");
  }
  return GPT_OK;
}

}  // namespace

template <typename T>
gpt_status launch_attn_fwd(const T* qkv, T* out, float* lse2, int B, int Tn, int H, int hd,
                           hipStream_t s) {
  const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
  dim3 grid(cdiv(Tn, 128), H, B);
  gpt_status st = dispatch_hd<T>(hd, [&](auto HD) {
    attn_fwd_kernel<T, decltype(HD)::value><<<grid, ATHREADS, 0, s>>>(qkv, out, lse2, Tn, H, sl2);
  });
  return st != GPT_OK ? st : check_launch("attention fwd");
}

template <typename T>
gpt_status launch_attn_bwd_stage(int stage, const T* qkv, const T* out, const T* dout,
                                 const float* lse2, float* dq_sum, T* dqkv, int B, int Tn, int H,
                                 int hd, hipStream_t s) {
  const float sl2 = 1.4426950408889634f / sqrtf((float)hd);
  const float scale = 1.f / sqrtf((float)hd);
  const long long N = (long long)B * Tn;
  dim3 grid(cdiv(Tn, 128), H, B);
  gpt_status st = dispatch_hd<T>(hd, [&](auto HD) {
    constexpr int hdv = decltype(HD)::value;
    if (stage == 0)
      attn_bwd_pre_kernel<T, hdv><<<cdiv(N * H, 256), 256, 0, s>>>(out, dout, dq_sum, N, Tn, H);
    else if (stage == 1)
      attn_bwd_dkdv_kernel<T, hdv><<<grid, ATHREADS, 0, s>>>(qkv, dout, lse2, dq_sum, dqkv, Tn, H,
                                                             sl2, scale);
    else
      attn_bwd_dq_kernel<T, hdv><<<grid, ATHREADS, 0, s>>>(qkv, dout, lse2, dq_sum, dqkv, Tn, H,
                                                           sl2, scale);
  });
  return st != GPT_OK ? st : check_launch("attention bwd");
}

template <typename T>
gpt_status launch_attn_bwd(const T* qkv, const T* out, const T* dout, const float* lse2,
                           float* dq_sum, T* dqkv, int B, int Tn, int H, int hd, hipStream_t s) {
  for (int stage = 0; stage < 3; ++stage) {
    gpt_status st = launch_attn_bwd_stage<T>(stage, qkv, out, dout, lse2, dq_sum, dqkv, B, Tn, H,
                                             hd, s);
    if (st != GPT_OK) return st;
  }
  return GPT_OK;
}

template gpt_status launch_attn_fwd<float>(const float*, float*, float*, int, int, int, int,
                                           hipStream_t);
template gpt_status launch_attn_fwd<bf16>(const bf16*, bf16*, float*, int, int, int, int,
                                          hipStream_t);
template gpt_status launch_attn_bwd<float>(const float*, const float*, const float*, const float*,
                                           float*, float*, int, int, int, int, hipStream_t);
template gpt_status launch_attn_bwd<bf16>(const bf16*, const bf16*, const bf16*, const float*,
                                          float*, bf16*, int, int, int, int, hipStream_t);
template gpt_status launch_attn_bwd_stage<float>(int, const float*, const float*, const float*,
                                                 const float*, float*, float*, int, int, int, int,
                                                 hipStream_t);
template gpt_status launch_attn_bwd_stage<bf16>(int, const bf16*, const bf16*, const bf16*,
                                                const float*, float*, bf16*, int, int, int, int,
                                                hipStream_t);

}  // namespace gpt
