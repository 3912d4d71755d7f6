// Internal helpers shared by the gfx950 kernels of libgpt: element types, vector loads,
// 64-wide wavefront reductions and the host-side status plumbing.
#pragma once

#include <vector>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "../../include/gpt.h"

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int WAVE = 64;

// ------------------------------------------------------------------ element helpers
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// Eight consecutive elements of T as one vector register group (16 B for bf16, 32 B for f32).
template <typename T> struct Vec8;
template <> struct Vec8<bf16> { typedef bf16x8 type; };
template <> struct Vec8<float> { typedef f32x8 type; };
template <typename T> using vec8_t = typename Vec8<T>::type;

template <typename T>
__device__ __forceinline__ vec8_t<T> load8(const T* p) {
  return *reinterpret_cast<const vec8_t<T>*>(p);
}
template <typename T>
__device__ __forceinline__ void store8(T* p, vec8_t<T> v) {
  *reinterpret_cast<vec8_t<T>*>(p) = v;
}
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float* out) {
  vec8_t<T> v = load8(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = to_f32(v[i]);
}
template <typename T>
__device__ __forceinline__ void store8_f32(T* p, const float* in) {
  vec8_t<T> v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = from_f32<T>(in[i]);
  store8(p, v);
}

// Buffer resource over [base, base + bytes) (bytes <= 2^31): raw loads at offsets past the end
// (OOB is one) read as zeros without touching memory, so loads need no per-lane branches.
constexpr uint32_t OOB = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x8 __attribute__((ext_vector_type(8)));
template <typename T>
__device__ __forceinline__ vec8_t<T> bload8(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(vec8_t<T>, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
  } else {
    const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16u, 0, 0);
    u32x8 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = lo[i];
      v[4 + i] = hi[i];
    }
    return __builtin_bit_cast(vec8_t<T>, v);
  }
}

// ------------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
  for (int o = width >> 1; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024); result valid in every thread.
__device__ __forceinline__ float block_sum(float v, float* smem /* >= 16 floats */) {
  v = wave_sum(v);
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE, nw = blockDim.x / WAVE;
  __syncthreads();
  if (l == 0) smem[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += smem[i];
  return t;
}
__device__ __forceinline__ float block_max(float v, float* smem) {
  v = wave_max(v);
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE, nw = blockDim.x / WAVE;
  __syncthreads();
  if (l == 0) smem[w] = v;
  __syncthreads();
  float t = -INFINITY;
  for (int i = 0; i < nw; ++i) t = fmaxf(t, smem[i]);
  return t;
}

// ------------------------------------------------------------------ host plumbing
namespace gpt {

void set_error(const std::string& msg);
gpt_status fail(gpt_status s, const std::string& msg);
gpt_status check_launch(const char* what);

inline unsigned cdiv(long long a, long long b) { return (unsigned)((a + b - 1) / b); }
inline size_t align_up(size_t n, size_t a = 256) { return (n + a - 1) / a * a; }

// Bump allocator over a caller-provided workspace: hands out consecutive 256-byte aligned
// regions (with a null base it only measures: size() is then the bytes a real carve needs).
// With `guard` set, every region is followed by a GUARD_BYTES guard region whose offset is
// recorded in `guards` (filled with a known pattern and checked later, so a kernel writing
// past the end of its buffer is detected).
constexpr size_t GUARD_BYTES = 256;
constexpr uint32_t GUARD_WORD = 0xA5C3F00Du;
struct Carver {
  char* base;
  size_t cap, off = 0;
  bool ok = true;
  bool guard = false;
  std::vector<size_t> guards;
  Carver(void* b, size_t c) : base((char*)b), cap(c) {}
  template <typename T>
  T* take(size_t n) {
    size_t at = align_up(off);
    off = at + n * sizeof(T);
    if (guard) {
      const size_t g = align_up(off);
      guards.push_back(g);
      off = g + GUARD_BYTES;
    }
    if (base == nullptr) return nullptr;
    if (off > cap) { ok = false; return nullptr; }
    return (T*)(base + at);
  }
  size_t size() const { return align_up(off); }
};

}  // namespace gpt
