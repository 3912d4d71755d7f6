// Softcapped cross-entropy forward + backward over bf16/fp32 logits (GPT.forward on the
// nanochat page: logits = 15 tanh(logits / 15), float cross-entropy with ignore_index -1,
// mean reduction).  One workgroup owns one token row: it reads the row once into registers,
// reduces the maximum and the sum of exponentials, and overwrites the row in place with
//   dz = (softmax(c) - onehot(target)) * (1 - tanh^2(z / cap)) * grad_scale / n_valid,
// so full-precision logits never exist in memory.  The per-row losses are summed in a fixed
// order by a single workgroup (deterministic).
#include "kernels.h"

#include <algorithm>

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
constexpr float LN2 = 0.6931471805599453f;

// 2^x and 1/x with the hardware instructions (v_exp_f32, v_rcp_f32: about 1 ulp).
__device__ __forceinline__ float hw_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float hw_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

typedef __fp16 h2 __attribute__((ext_vector_type(2)));

// Per-thread storage of q = exp(c - running max) * (1 - th^2): packed fp16 pairs for bf16 logits
// (q is in [0, 1]; fp16 keeps 11 bits, more than the bf16 gradient that is stored from it), fp32
// pairs for fp32 logits.
template <typename T> struct EStore;
// pin() is an empty asm use: the value is computed by that point, which keeps the optimizer from
// sinking each piece's math below the next row's loads (both rows' logits would then be live).
template <> struct EStore<bf16> {
  h2 v;
  __device__ __forceinline__ void set(float a, float b) { v = __builtin_amdgcn_cvt_pkrtz(a, b); }
  __device__ __forceinline__ float get(int i) const { return (float)v[i]; }
  __device__ __forceinline__ void pin() const { asm volatile("" ::"v"(v)); }
};
template <> struct EStore<float> {
  float v[2];
  __device__ __forceinline__ void set(float a, float b) { v[0] = a; v[1] = b; }
  __device__ __forceinline__ float get(int i) const { return v[i]; }
  __device__ __forceinline__ void pin() const { asm volatile("" ::"v"(v[0]), "v"(v[1])); }
};

// Largest raw logit of a thread.  bf16 values are compared as 16-bit integer keys (sign-magnitude
// turned into two's-complement order: negative values get their magnitude bits flipped), two per
// packed max, so the maximum pass does not convert the values to fp32 (the compiler would keep
// those 128 conversions alive for the main pass).
typedef short s16x2 __attribute__((ext_vector_type(2)));
struct RawMaxBf16 {
  s16x2 k = {-32767, -32767};
  __device__ __forceinline__ void add(const bf16x8& v, bool live) {
    const u32x4 w = __builtin_bit_cast(u32x4, v);
    const s16x2 none = {-32767, -32767};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // (a bit_cast of the subscript w[i] itself reads element 0 with this compiler: copy first)
      const unsigned int wi = w[i];
      const s16x2 x = __builtin_bit_cast(s16x2, wi);
      k = __builtin_elementwise_max(k, live ? x ^ ((x >> (short)15) & (short)0x7FFF) : none);
    }
  }
  __device__ __forceinline__ float get() const {
    const short m = k[0] > k[1] ? k[0] : k[1];
    const short b = m ^ ((m >> 15) & 0x7FFF);
    return __builtin_bit_cast(float, (uint32_t)(uint16_t)b << 16);
  }
};
struct RawMaxF32 {
  float m = -3.402823466e38f;
  __device__ __forceinline__ void add(const f32x8& v, bool live) {
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, live ? v[i] : -3.402823466e38f);
  }
  __device__ __forceinline__ float get() const { return m; }
};
template <typename T> struct RawMax;
template <> struct RawMax<bf16> { typedef RawMaxBf16 type; };
template <> struct RawMax<float> { typedef RawMaxF32 type; };

// Lowest finite float: the starting maximum, so that combining two empty partials gives 0, not NaN.
constexpr float NEG_BIG = -3.402823466e38f;

// Combines (m, s) partials over the block: m = max of the m's, s = sum of s * 2^(m_i - m), with
// one LDS exchange through smem[0 .. 2 * TH/64).
template <int TH>
__device__ __forceinline__ void block_max_sum(float& m, float& s, float* smem) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float mo = __shfl_xor(m, o, WAVE), so = __shfl_xor(s, o, WAVE);
    const float mn = fmaxf(m, mo);
    s = s * hw_exp2(m - mn) + so * hw_exp2(mo - mn);
    m = mn;
  }
  constexpr int NW = TH / WAVE;
  const int w = threadIdx.x / WAVE;
  if (threadIdx.x % WAVE == 0) {
    smem[w] = m;
    smem[NW + w] = s;
  }
  __syncthreads();
  float M = NEG_BIG;
#pragma unroll
  for (int i = 0; i < NW; ++i) M = fmaxf(M, smem[i]);
  float S = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) S += smem[NW + i] * hw_exp2(smem[i] - M);
  m = M;
  s = S;
}

// The row's pieces of 8 columns that thread x holds: columns 8 (x + gi TH) .. +7, gi < G.  Pieces
// past the row (and every piece of a row index past the last) read zeros through the buffer
// resource, with no memory access and no per-lane branch.
template <typename T, int TH, int G>
__device__ __forceinline__ void load_row(vec8_t<T> (&raw)[G], const T* zr, bool live, int V) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(zr, live ? (uint32_t)((size_t)V * sizeof(T)) : 0u);
  const int groups = V / 8;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int g = threadIdx.x + gi * TH;
    raw[gi] = bload8<T>(rs, g < groups ? (uint32_t)(g * 8 * sizeof(T)) : OOB);
  }
}

// Element i of a row of V (0 when i is outside [0, V)), through a buffer resource: no branch, so
// the compiler can count it among the outstanding loads.
template <typename T>
__device__ __forceinline__ T load_one(const T* zr, int i, int V) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(zr, (uint32_t)((size_t)V * sizeof(T)));
  const uint32_t off = i >= 0 && i < V ? (uint32_t)(i * sizeof(T)) : OOB;
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
  } else {
    return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  }
}

// Stores 8 values (rounded to T) at byte offset off of the resource (dropped at OOB).
template <typename T>
__device__ __forceinline__ void bstore8(__amdgpu_buffer_rsrc_t rs, uint32_t off, const float* d) {
  vec8_t<T> v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = from_f32<T>(d[i]);
  if constexpr (sizeof(T) == 2) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, 0);
  } else {
    const u32x8 w = __builtin_bit_cast(u32x8, v);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[0], w[1], w[2], w[3]}, rs, off, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{w[4], w[5], w[6], w[7]}, rs, off + 16u, 0, 0);
  }
}

// Stores one value (rounded to T) at byte offset off of the resource.
template <typename T>
__device__ __forceinline__ void bstore1(__amdgpu_buffer_rsrc_t rs, uint32_t off, float x) {
  if constexpr (sizeof(T) == 2) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, from_f32<T>(x)), rs, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned int, x), rs, off, 0, 0);
  }
}

// Rows r = blockIdx.x, blockIdx.x + gridDim.x, ... of the logits, one workgroup at a time, each
// overwritten in place with its gradient.  In base-2 units (c2 = c log2 e, c = cap * tanh(z / cap)
// or z), the thread's maximum m_t comes from its largest raw logit (c is increasing in z), so each
// column is visited once:
//   e = 2^(c2 - m_t),  s_t = sum e,  q = e * (1 - th^2)      (1 - th^2 = dc/dz; 1 without a cap)
// and only q is kept (one packed value per column).  The block combines M = max m_t and
// S = sum s_t 2^(m_t - M), so lse = (M + log2 S) ln 2, and the gradient is
//   dz = q * 2^(m_t - M) / S * scale  -  [target] (1 - th_t^2) * scale,
// with the one-hot term applied by the lane that owns the target column.  The next row's loads
// are issued as soon as the current row's logits are consumed, so they are in flight during
// this row's reduction, gradient and stores.
template <typename T, int TH, int G, bool CAPPED>
__global__ __launch_bounds__(TH, 2) void ce_kernel(T* __restrict__ z, long long ldz,
                                                  const int32_t* __restrict__ tgt, long long rows,
                                                  int V, float cap, float grad_scale,
                                                  const int* __restrict__ n_valid,
                                                  float* __restrict__ loss_rows) {
  __shared__ float smem[2][2 * TH / WAVE];  // reduction slots, alternating between rows
  const int groups = V / 8;
  const int nv = *n_valid;
  const float k2 = CAPPED ? 2.f * LOG2E / cap : 0.f;  // exp(2 z / cap) = 2^(z * k2)
  const float c2mul = CAPPED ? cap * LOG2E : LOG2E;    // c2 = c2mul * th
  auto tanh_cap = [&](float x) { return CAPPED ? 1.f - 2.f * hw_rcp(hw_exp2(x * k2) + 1.f) : x; };
  long long row = blockIdx.x;
  if (row >= rows) return;
  const long long stride = gridDim.x;
  // the row's logits and its target logit are loaded one row ahead, its target index two ahead
  vec8_t<T> raw[G];
  int t = tgt[row];
  int t_next = tgt[row + stride < rows ? row + stride : row];
  T zt = load_one<T>(z + row * ldz, t, V);
  load_row<T, TH, G>(raw, z + row * ldz, true, V);
  float mt, s, c2t, dt;  // thread maximum and sum; target column c log2 e and dc/dz (uniform)
  EStore<T> q[G][4];
  auto consume = [&]() {
    const float th_t = tanh_cap(to_f32(zt));
    c2t = c2mul * th_t;
    dt = CAPPED ? fmaf(-th_t, th_t, 1.f) : 1.f;
    typename RawMax<T>::type xm;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) xm.add(raw[gi], (int)threadIdx.x + gi * TH < groups);
    // a thread with no columns (only for rows narrower than the block) contributes s = 0
    mt = (int)threadIdx.x < groups ? c2mul * tanh_cap(xm.get()) : NEG_BIG;
    s = 0.f;
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int g = threadIdx.x + gi * TH;
      float ex[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float th = tanh_cap(to_f32(raw[gi][e]));
        ex[e] = hw_exp2(c2mul * th - mt);
        s += g < groups ? ex[e] : 0.f;
        if (CAPPED) ex[e] *= fmaf(-th, th, 1.f);
      }
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        q[gi][k].set(ex[2 * k], ex[2 * k + 1]);
        q[gi][k].pin();
      }
    }
    // the sum is complete (so is every q) before the next row's loads reuse the registers
    asm volatile("" ::"v"(s) : "memory");
  };
  consume();
  for (int it = 0;; ++it) {
    const bool valid = t >= 0 && t < V;
    const long long next = row + stride;
    const long long next2 = next + stride;
    const int t_next2 = tgt[next2 < rows ? next2 : row];
    load_row<T, TH, G>(raw, z + next * ldz, next < rows, V);
    const T zt_next = load_one<T>(z + next * ldz, next < rows ? t_next : -1, V);
    float M = mt, S = s;
    block_max_sum<TH>(M, S, smem[it & 1]);
    const float scale = valid ? grad_scale / (float)(nv > 0 ? nv : 1) : 0.f;
    const float F = hw_exp2(mt - M) * (scale / S);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(z + row * ldz, (uint32_t)((size_t)V * sizeof(T)));
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const int g = threadIdx.x + gi * TH;
      float d[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) d[e] = q[gi][e / 2].get(e % 2) * F;
      bstore8<T>(rs, g < groups ? (uint32_t)(g * 8 * sizeof(T)) : OOB, d);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the target column, rewritten by the lane that stored it (program order within the lane):
    // (softmax - 1) * dc/dz * scale
    if (valid && (int)threadIdx.x == (t / 8) % TH) {
      const float dtgt = (hw_exp2(c2t - M) / S - 1.f) * dt * scale;
      bstore1<T>(rs, (uint32_t)(t * sizeof(T)), dtgt);
    }
    if (threadIdx.x == 0) loss_rows[row] = valid ? (M + __log2f(S) - c2t) * LN2 : 0.f;
    if (next >= rows) break;
    row = next;
    t = t_next;
    t_next = t_next2;
    zt = zt_next;
    consume();
  }
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

// Workgroups of `kernel` that fit one CU times the device's CUs (cached per kernel and device).
template <class K>
unsigned resident_grid(K kernel, int threads) {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu <= 0) per_cu = 1;
    cached[dev] = cus * per_cu;
  }
  return (unsigned)cached[dev];
}

template <typename T>
gpt_status launch_ce(T* z, long long ldz, const int32_t* tgt, long long rows, int V, float cap,
                     float grad_scale, const int* n_valid, float* loss_rows, hipStream_t s) {
  if (rows == 0) return GPT_OK;
  // Each of the row's V/8 pieces of 8 columns lives in one thread's registers (at most G per
  // thread); a resident grid walks the rows.
  const int g = V / 8;
#define CE_LAUNCH(TH, G, CAPPED)                                                               \
  do {                                                                                         \
    auto k = ce_kernel<T, TH, G, CAPPED>;                                                      \
    const unsigned grid = (unsigned)std::min<long long>(rows, resident_grid(k, TH));          \
    k<<<grid, TH, 0, s>>>(z, ldz, tgt, rows, V, cap, grad_scale, n_valid, loss_rows);          \
  } while (0)
#define CE_CASE(TH, G)                        \
  do {                                        \
    if (cap > 0.f) CE_LAUNCH(TH, G, true);    \
    else CE_LAUNCH(TH, G, false);             \
  } while (0)
  if (g <= 256) CE_CASE(256, 1);
  else if (g <= 1024) CE_CASE(256, 4);
  else if (g <= 2048) CE_CASE(256, 8);
  else if (g <= 4096) CE_CASE(512, 8);
  else if (g <= 6656) CE_CASE(512, 13);  // V <= 53,248 (GPT-2's 50,304: 94% of the slots used)
  else if (g <= 8192) CE_CASE(1024, 8);  // 16 waves: 827 -> 793 us at 16384 x 65536 (512 x 16)
  else return fail(GPT_ESHAPE, "vocab above 65536 is not supported");
#undef CE_CASE
#undef CE_LAUNCH
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
