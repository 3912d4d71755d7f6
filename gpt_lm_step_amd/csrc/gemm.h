// GEMM launcher and its fused epilogues (internal to libgpt).
#pragma once

#include "kernels.h"

namespace gpt {

// out = T(acc)
template <typename T>
struct EpiStore {
  T* out;
  long long ldo;
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    out[(long long)r * ldo + c] = from_f32<T>(v);
  }
};

// out = acc, or out += acc when beta != 0 (fp32 gradients, accumulation across calls).
struct EpiStoreF32 {
  float* out;
  long long ldo;
  int beta;
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    float* p = out + (long long)r * ldo + c;
    *p = beta ? *p + v : v;
  }
};

// out = res + acc (fp32 residual stream; out may equal res).
struct EpiResid {
  const float* res;
  float* out;
  long long ld;
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    const long long i = (long long)r * ld + c;
    out[i] = res[i] + v;
  }
};

// q/k/v projection: columns >= vcol0 (the values) get the per-token addend u (fp32).
template <typename T>
struct EpiQKV {
  T* out;
  long long ldo;
  const float* u;
  long long ldu;
  int vcol0;
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    if (u && c >= vcol0) v += u[(long long)r * ldu + (c - vcol0)];
    out[(long long)r * ldo + c] = from_f32<T>(v);
  }
};

// MLP up projection: hp = acc, act = relu(acc)^2.
template <typename T>
struct EpiRelu2 {
  T* hp;
  T* act;
  long long ld;
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    const long long i = (long long)r * ld + c;
    hp[i] = from_f32<T>(v);
    const float m = v > 0.f ? v : 0.f;
    act[i] = from_f32<T>(m * m);
  }
};

// Down-projection input gradient through ReLU^2: out = acc * 2 * relu(hp).
template <typename T>
struct EpiDRelu2 {
  const T* hp;
  T* out;
  long long ld;
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    const long long i = (long long)r * ld + c;
    const float h = to_f32(hp[i]);
    out[i] = from_f32<T>(h > 0.f ? 2.f * h * v : 0.f);
  }
};

// out (fp32) = acc + add (add in T, optional): the value addend u = v_add + tri * wtri^T.
template <typename T>
struct EpiAddRows {
  const T* add;
  float* out;
  long long ld;
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    const long long i = (long long)r * ld + c;
    out[i] = v + (add ? to_f32(add[i]) : 0.f);
  }
};

// C[m,n] = sum_k A(m,k) B(n,k); a_kc/b_kc select K-contiguous (p[r*ld+k]) or row-contiguous
// (p[k*ld+r]) operands.  Requirements: K % 8 == 0, lda/ldb % 8 == 0, 16-byte aligned operands,
// M % 8 == 0 for a row-contiguous A and N % 8 == 0 for a row-contiguous B.
template <typename T, class Epi>
gpt_status gemm(bool a_kc, bool b_kc, int M, int N, int K, const T* A, long long lda, const T* B,
                long long ldb, const Epi& epi, hipStream_t s);

}  // namespace gpt
