// Matrix-core GEMMs of the step (q/k/v, out, MLP up/down and LM-head projections and their
// input- and weight-gradients, the Newton-Schulz products of the optimizer, the prefill
// products of inference), hand-written for gfx950.
//
//   C[m, n] = sum_k A(m, k) * B(n, k)
//
// Each operand is either K-contiguous ("KC": element (r, k) at p[r*ld + k]) or row-contiguous
// ("RC": element (r, k) at p[k*ld + r]).  Forward projections y = x W^T are KC x KC; input
// gradients dx = dy W are KC x RC; weight gradients dW = dy^T x are RC x RC.
//
// bf16 (gemm_dma_kernel): one workgroup per 256 x 256 output tile (8 waves, two per SIMD, each
// 128 x 64 or 64 x 128) when that tiling has enough tiles to fill the GPU, else 128 x 128 (4
// waves, two workgroups per CU):
//  * operand tiles travel global -> LDS by LDS-DMA buffer loads in the operand's own layout
//    (XOR-swizzled, no staging registers, no LDS store instructions); RC tiles are read back
//    with transposing LDS reads; loads past an operand's end read zeros (buffer range check);
//  * K advances through a ring of LDS stages: two 64-wide stages when A is K-contiguous (whole
//    128-byte lines per DMA row), four 32-wide stages otherwise; one barrier per K tile, the
//    next tile's first fragments read during the current tile's last MFMAs;
//  * v_mfma_f32_32x32x16_bf16 with the B fragment first, so each lane ends with 4 consecutive
//    output columns; the epilogue stages 32-row slices through LDS and stores coalesced rows;
//  * epilogues are fused: bf16/fp32 stores, value addend, rotary + QK-norm (EpiQKVRope), ReLU^2,
//    dReLU^2, residual add, beta-accumulation, split-K partials, Newton-Schulz combinations;
//  * blocks are dispatched round-robin over the 8 XCDs; each XCD walks a contiguous range of
//    tiles in groups of 4 row tiles (operand panels shared in its L2);
//  * shapes whose tiling leaves CUs idle and that have an fp32 output (weight gradients, the LM
//    head's input gradient) split K into fp32 partials reduced in split order (deterministic);
//  * two independent weight gradients whose tiles together make one round of the CUs can run as
//    one paired launch (gemm_wgrad_pair).
// fp32 (gemm_kernel, the parity configurations only): 64 x 64 tiles staged through registers.
// Header-only: every call site instantiates its own kernel symbol (a GemmSite tag), so
// profiles name the projection a launch belongs to.
#pragma once

#include <type_traits>
#include <utility>

#include "kernels.h"

namespace gpt {

// Epilogues receive 4 consecutive columns c..c+3 of one output row r (c is a multiple of 4).
template <typename T> struct Vec4T;
template <> struct Vec4T<bf16> { typedef bf16x4 type; };
template <> struct Vec4T<float> { typedef f32x4 type; };
template <typename T> using vec4t = typename Vec4T<T>::type;

template <typename T>
__device__ __forceinline__ void store4(T* p, const float (&v)[4]) {
  vec4t<T> o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = from_f32<T>(v[i]);
  // streaming store: every CU writes its tile at about the same time, and the non-temporal hint
  // drains that burst faster (measured 141 -> 117 us of fixed cost on 16384 x 8192 outputs)
  __builtin_nontemporal_store(o, reinterpret_cast<vec4t<T>*>(p));
}
template <typename T>
__device__ __forceinline__ void load4(const T* p, float (&v)[4]) {
  const vec4t<T> x = *reinterpret_cast<const vec4t<T>*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = to_f32(x[i]);
}

// Each epilogue is split into load(r, c), which fetches what the output depends on besides the
// accumulator (nothing for plain stores), and store(r, c, v, pre).  The tiled kernels issue the
// loads of all their row passes before the first store, so the load latencies overlap instead of
// being paid one after another (the compiler cannot reorder a load after a store that may
// alias it).  operator() is the two in sequence.
struct NoPre {};
template <typename T>
struct Pre4 {
  vec4t<T> x;
};
template <typename T>
__device__ __forceinline__ Pre4<T> pre_load(const T* p) {
  return Pre4<T>{*reinterpret_cast<const vec4t<T>*>(p)};
}
template <typename T>
__device__ __forceinline__ void pre_add(const Pre4<T>& a, float (&o)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] += to_f32(a.x[i]);
}
#define GPT_EPI_CALL                                                                     \
  __device__ __forceinline__ void operator()(int r, int c, const float (&v)[4]) const { \
    store(r, c, v, load(r, c));                                                          \
  }

// out = T(acc)
template <typename T>
struct EpiStore {
  T* out;
  long long ldo;
  using Pre = NoPre;
  __device__ __forceinline__ Pre load(int, int) const { return {}; }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre&) const {
    store4(out + (long long)r * ldo + c, v);
  }
  GPT_EPI_CALL
};

// fp32 output descriptor: out = acc, or out += acc when beta != 0 (gradients accumulated across
// calls).  gemm() launches it as EpiPutF32 or EpiAccF32, so no kernel branches on beta.
struct EpiStoreF32 {
  float* out;
  long long ldo;
  int beta;
};
struct EpiPutF32 {
  float* out;
  long long ldo;
  using Pre = NoPre;
  __device__ __forceinline__ Pre load(int, int) const { return {}; }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre&) const {
    store4(out + (long long)r * ldo + c, v);
  }
  GPT_EPI_CALL
};
struct EpiAccF32 {
  float* out;
  long long ldo;
  using Pre = Pre4<float>;
  __device__ __forceinline__ Pre load(int r, int c) const {
    return pre_load(out + (long long)r * ldo + c);
  }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre& a) const {
    float o[4] = {v[0], v[1], v[2], v[3]};
    pre_add(a, o);
    store4(out + (long long)r * ldo + c, o);
  }
  GPT_EPI_CALL
};

// Split-K partial: split blockIdx.y of the K range writes its fp32 [M][N] sum at
// ws + blockIdx.y * stride (row pitch N).
struct EpiSplit {
  float* ws;
  long long stride, ldo;
  using Pre = NoPre;
  __device__ __forceinline__ Pre load(int, int) const { return {}; }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre&) const {
    store4(ws + blockIdx.y * stride + (long long)r * ldo + c, v);
  }
  GPT_EPI_CALL
};

// out = res + acc (fp32 residual stream; out may equal res).
// Batched bf16 products of the Newton-Schulz iteration (matrix z of a batch at out + z * bs):
// a plain store, and out = alpha * acc + beta * add with `add` in the output's layout.  With SYM
// the product is known to be symmetric (X X^T, c A A + b A for symmetric A): the kernel computes
// the upper-triangle tiles only and mirror_col() writes each off-diagonal tile's values
// transposed, one mirrored row run of 32 per lane read back from the staged tile.
template <bool SYM>
struct EpiNsStoreT {
  bf16* out;
  long long ld, bs;
  using Pre = NoPre;
  static constexpr bool symmetric = SYM;
  __device__ __forceinline__ void at_batch(int z) { out += (long long)z * bs; }
  __device__ __forceinline__ Pre load(int, int) const { return {}; }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre&) const {
    store4(out + (long long)r * ld + c, v);
  }
  // the mirrored run: out[c][r0 .. r0+31] = v[0 .. 31] (v = column c of rows r0..r0+31)
  __device__ __forceinline__ void mirror_col(int r0, int c, const float (&v)[32]) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float o[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = v[q * 8 + e];
      store8_f32(out + (long long)c * ld + r0 + q * 8, o);
    }
  }
  GPT_EPI_CALL
};
template <bool SYM>
struct EpiNsCombineT {
  bf16* out;
  const bf16* add;
  long long ld, bs;
  float alpha, beta;
  using Pre = Pre4<bf16>;
  static constexpr bool symmetric = SYM;
  __device__ __forceinline__ void at_batch(int z) {
    out += (long long)z * bs;
    add += (long long)z * bs;
  }
  __device__ __forceinline__ Pre load(int r, int c) const {
    return pre_load(add + (long long)r * ld + c);
  }
  __device__ __forceinline__ void combine(const float (&v)[4], const Pre& a, float (&o)[4]) const {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = alpha * v[i] + beta * to_f32(a.x[i]);
  }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre& a) const {
    float o[4];
    combine(v, a, o);
    store4(out + (long long)r * ld + c, o);
  }
  // the mirrored run: out[c][r0 .. r0+31] = alpha v + beta add[c][r0 ..] (add is symmetric, so
  // its mirrored entries equal the ones the direct store used)
  __device__ __forceinline__ void mirror_col(int r0, int c, const float (&v)[32]) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float a8[8], o[8];
      load8_f32(add + (long long)c * ld + r0 + q * 8, a8);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = alpha * v[q * 8 + e] + beta * a8[e];
      store8_f32(out + (long long)c * ld + r0 + q * 8, o);
    }
  }
  GPT_EPI_CALL
};
using EpiNsStore = EpiNsStoreT<false>;
using EpiNsCombine = EpiNsCombineT<false>;
using EpiNsStoreSym = EpiNsStoreT<true>;
using EpiNsCombineSym = EpiNsCombineT<true>;

struct EpiResid {
  const float* res;
  float* out;
  long long ld;
  using Pre = Pre4<float>;
  __device__ __forceinline__ Pre load(int r, int c) const {
    return pre_load(res + (long long)r * ld + c);
  }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre& a) const {
    float o[4] = {v[0], v[1], v[2], v[3]};
    pre_add(a, o);
    store4(out + (long long)r * ld + c, o);
  }
  GPT_EPI_CALL
};

// q/k/v projection: columns >= vcol0 (the values) get the per-token addend u (fp32).  gemm()
// launches a plain EpiStore when u is null.
template <typename T>
struct EpiQKV {
  T* out;
  long long ldo;
  const float* u;
  long long ldu;
  int vcol0;
  using Pre = Pre4<float>;
  __device__ __forceinline__ Pre load(int r, int c) const {
    // columns left of vcol0 read the row's first addend entries and ignore them
    return pre_load(u + (long long)r * ldu + max(c - vcol0, 0));
  }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre& a) const {
    float o[4] = {v[0], v[1], v[2], v[3]};
    if (c >= vcol0) pre_add(a, o);
    store4(out + (long long)r * ldo + c, o);
  }
  GPT_EPI_CALL
};

// q/k/v projection with the rotary embedding and the QK-norm applied in the epilogue (the
// rotation and per-head RMSNorm of CausalSelfAttention.forward on the nanochat page, as
// rope_qknorm_fwd_kernel computes them, but on the fp32 accumulator instead of a stored bf16
// product).  Columns [0, D) are q, [D, 2D) k, [2D, 3D) v, head h of a block at h * hd.  For q
// and k: with t = r mod T and i = column mod hd/2, the first half of a head becomes
// x1 cos_i + x2 sin_i and the second -x1 sin_i + x2 cos_i; the kernel hands each lane four
// such pairs of one row (columns c..c+3 and c+hd/2..), hd/8 lanes per head.  With QKN every
// head is then scaled by r = 1/sqrt(mean(y^2) + eps) and r is saved in rstd_qk [N, 2H] (q
// heads, then k heads).  v columns get the value addend u (VADD) as EpiQKV does.  Requires
// wave tiles whose column span is a multiple of hd starting at a multiple of hd, and D a
// multiple of 128, so that every column test below is wave-uniform.
template <typename T, bool QKN, bool VADD>
struct EpiQKVRope {
  T* out;
  long long ldo;
  const T* cos_t;
  const T* sin_t;
  float* rstd_qk;
  const float* u;
  long long ldu;
  int D, hd, Tn, H;
  float eps;
  static constexpr int wave_cols = 128;  // wave tiles of 128 columns (a head of up to 128)
  static constexpr bool pairs = true;    // the kernel hands over rotation pairs (see below)
  struct Pre {
    vec4t<T> c, s;
    f32x4 u1, u2;
  };
  // Row r; c: column of the first element of four in a head's first half (c2 = c + hd/2 holds
  // their rotation partners).
  __device__ __forceinline__ Pre load(int r, int c) const {
    Pre p;
    const int half = hd / 2, i = c % hd, t = r % Tn;
    p.c = *reinterpret_cast<const vec4t<T>*>(cos_t + (long long)t * half + i);
    p.s = *reinterpret_cast<const vec4t<T>*>(sin_t + (long long)t * half + i);
    if constexpr (VADD) {
      // q and k columns read the row's first addend entries and ignore them
      const float* ur = u + (long long)r * ldu + max(c - 2 * D, 0);
      p.u1 = *reinterpret_cast<const f32x4*>(ur);
      p.u2 = *reinterpret_cast<const f32x4*>(ur + (c >= 2 * D ? half : 0));
    }
    return p;
  }
  __device__ __forceinline__ void store(int r, int c, const float (&x1)[4], const float (&x2)[4],
                                        const Pre& a) const {
    float y1[4], y2[4];
    const int c2 = c + hd / 2;
    if (c < 2 * D) {  // wave-uniform
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float cs = to_f32(a.c[e]), sn = to_f32(a.s[e]);
        y1[e] = x1[e] * cs + x2[e] * sn;
        y2[e] = -x1[e] * sn + x2[e] * cs;
        ss += y1[e] * y1[e] + y2[e] * y2[e];
      }
      if constexpr (QKN) {
        ss = group_sum(ss, hd / 8);
        const float rs = 1.f / sqrtf(ss / (float)hd + eps);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y1[e] *= rs;
          y2[e] *= rs;
        }
        if (c % hd == 0) rstd_qk[(long long)r * 2 * H + c / hd] = rs;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        y1[e] = x1[e];
        y2[e] = x2[e];
      }
      if constexpr (VADD) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          y1[e] += a.u1[e];
          y2[e] += a.u2[e];
        }
      }
    }
    store4(out + (long long)r * ldo + c, y1);
    store4(out + (long long)r * ldo + c2, y2);
  }
};

// MLP up projection: act = relu(acc)^2 (the only activation the backward needs: the derivative
// 2 relu(h) equals 2 sqrt(act)).
template <typename T>
struct EpiRelu2 {
  T* act;
  long long ld;
  using Pre = NoPre;
  __device__ __forceinline__ Pre load(int, int) const { return {}; }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre&) const {
    float a[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float m = v[k] > 0.f ? v[k] : 0.f;
      a[k] = m * m;
    }
    store4(act + (long long)r * ld + c, a);
  }
  GPT_EPI_CALL
};

// Down-projection input gradient through ReLU^2: out = acc * 2 relu(h) = acc * 2 sqrt(act).
template <typename T>
struct EpiDRelu2 {
  const T* act;
  T* out;
  long long ld;
  using Pre = Pre4<T>;
  __device__ __forceinline__ Pre load(int r, int c) const {
    return pre_load(act + (long long)r * ld + c);
  }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre& a) const {
    float o[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float x = to_f32(a.x[k]);
      o[k] = x > 0.f ? 2.f * __builtin_amdgcn_sqrtf(x) * v[k] : 0.f;
    }
    store4(out + (long long)r * ld + c, o);
  }
  GPT_EPI_CALL
};

// out (fp32) = acc + add (add in T, optional: gemm() launches EpiPutF32 when it is null): the
// value addend u = v_add + tri * wtri^T.
template <typename T>
struct EpiAddRows {
  const T* add;
  float* out;
  long long ld;
  using Pre = Pre4<T>;
  __device__ __forceinline__ Pre load(int r, int c) const {
    return pre_load(add + (long long)r * ld + c);
  }
  __device__ __forceinline__ void store(int r, int c, const float (&v)[4], const Pre& a) const {
    float o[4] = {v[0], v[1], v[2], v[3]};
    pre_add(a, o);
    store4(out + (long long)r * ld + c, o);
  }
  GPT_EPI_CALL
};
#undef GPT_EPI_CALL

// Call sites of the GEMM: each gets its own kernel symbol, so profiles name the projection.
enum GemmSite {
  G_TEST = 0, G_QKV, G_OUT, G_UP, G_DOWN, G_HEAD, G_HEAD_DGRAD, G_HEAD_WGRAD, G_DOWN_DGRAD,
  G_DOWN_WGRAD, G_UP_DGRAD, G_UP_WGRAD, G_OUT_DGRAD, G_OUT_WGRAD, G_QKV_DGRAD, G_QKV_WGRAD,
  G_TRI, G_TRI_WGRAD, G_NS_GRAM, G_NS_POLY, G_NS_APPLY, G_INF_QKV, G_INF_OUT, G_INF_UP,
  G_INF_DOWN, G_INF_HEAD, G_QKV_OUT_WGRAD
};

// Passes of an epilogue row slice whose loads may be in flight together (Epi::pass_group when
// the epilogue declares one, else all of them), and the wave-tile column span it needs
// (Epi::wave_cols, else the default 64).
template <class E, class = void>
struct epi_pg : std::integral_constant<int, 32> {};
template <class E>
struct epi_pg<E, std::void_t<decltype(E::pass_group)>> : std::integral_constant<int, E::pass_group> {};
template <class E>
constexpr int epi_pass_group() { return epi_pg<E>::value; }
template <class E, class = void>
struct epi_pairs : std::false_type {};
template <class E>
struct epi_pairs<E, std::enable_if_t<E::pairs>> : std::true_type {};
template <class E, class = void>
struct epi_wave_cols : std::integral_constant<int, 64> {};
template <class E>
struct epi_wave_cols<E, std::void_t<decltype(E::wave_cols)>> : std::integral_constant<int, E::wave_cols> {};

// Epilogues of products known to be symmetric (see EpiNsStoreT).
template <class E, class = void>
struct is_symmetric : std::false_type {};
template <class E>
struct is_symmetric<E, std::enable_if_t<E::symmetric>> : std::true_type {};

namespace gemm_detail {

constexpr int THREADS = 256;  // 4 waves in a 2 x 2 grid; each wave owns a (BM/2) x (BN/2) tile

template <typename T> struct Mma;
template <> struct Mma<bf16> {
  static __device__ __forceinline__ void run(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
  }
};
template <> struct Mma<float> {
  static __device__ __forceinline__ void run(f32x16& acc, const f32x8& a, const f32x8& b) {
#pragma unroll
    for (int s = 0; s < 8; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
  }
};

template <typename T>
struct Cfg {
  static constexpr int BK = 128 / sizeof(T);              // 128 bytes of K per tile row
  static constexpr int PITCH = BK + 16 / sizeof(T);       // +16 B padding per LDS row
  static constexpr int KV = BK / 8;                       // 8-element vectors per tile row
};

// Global -> registers -> LDS staging of one ROWS x BK operand tile.  KC tiles: thread v moves
// 16 B vector v (row v / KV, chunk v % KV).  RC tiles: thread t moves the 8 x 8 block
// (k-chunk t % (BK/8), row block t / (BK/8)): each global load instruction still reads whole
// 128-byte row segments, and the transposed LDS writes of neighbouring threads fall in distinct
// banks (row pitch 144 B).
template <typename T, int ROWS, bool KC>
struct Stage {
  using C = Cfg<T>;
  using V = vec8_t<T>;
  static constexpr int NVEC = ROWS * C::KV;                       // KC: vectors per tile
  static constexpr int NBLK = (C::BK / 8) * (ROWS / 8);           // RC: 8x8 blocks per tile
  static constexpr int PER = KC ? (NVEC + THREADS - 1) / THREADS : 8 * ((NBLK + THREADS - 1) / THREADS);
  V r[PER];

  // Branch-free loads through a buffer resource: an element outside [0, rows_lim) x [0, k_lim)
  // gets an offset past the resource's end, which the hardware returns as zeros.
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t rs, long long ld, int row0, int k0,
                                       int rows_lim, int k_lim) {
    const int tid = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int v = tid + i * THREADS;
        const int row = row0 + v / C::KV, k = k0 + (v % C::KV) * 8;
        const bool ok = v < NVEC && row < rows_lim && k < k_lim;
        r[i] = bload8<T>(rs, ok ? (uint32_t)(((long long)row * ld + k) * sizeof(T)) : OOB);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER / 8; ++j) {
        const int blk = tid + j * THREADS;
        const int kb = blk % (C::BK / 8), rb = blk / (C::BK / 8);
        const int row = row0 + rb * 8;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int k = k0 + kb * 8 + kk;
          const bool ok = blk < NBLK && row < rows_lim && k < k_lim;
          r[j * 8 + kk] = bload8<T>(rs, ok ? (uint32_t)(((long long)k * ld + row) * sizeof(T)) : OOB);
        }
      }
    }
  }

  __device__ __forceinline__ void store(T* lds) const {
    const int tid = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int v = tid + i * THREADS;
        if (NVEC % THREADS == 0 || v < NVEC) store8(lds + (v / C::KV) * C::PITCH + (v % C::KV) * 8, r[i]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < PER / 8; ++j) {
        const int blk = tid + j * THREADS;
        if (NBLK % THREADS != 0 && blk >= NBLK) continue;
        const int kb = blk % (C::BK / 8), rb = blk / (C::BK / 8);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          V o;
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) o[kk] = r[j * 8 + kk][rr];
          store8(lds + (rb * 8 + rr) * C::PITCH + kb * 8, o);
        }
      }
    }
  }
};

// Logical tile order: blocks are dispatched round-robin over the 8 XCDs, so block b runs on
// XCD b % 8.  Give XCD x the contiguous range of logical tiles x*per .. x*per+per-1, and walk
// tiles in groups of GROUP_M row-tiles so that consecutive tiles share A and B panels.  Groups
// of 4 measured best on the d32 products (against 8: dReLU^2 dgrad 549 -> 522-529 us, out
// dgrad 128 -> 121-124 us, down projection 546-555 -> 534-541 us; 2 about the same as 4, 1 and
// 16 slower) and neutral on GPT-2-small's.
// Block b of nb blocks (a paired launch numbers each problem's blocks from 0; its first
// problem's block count is a multiple of 8, so block b still runs on XCD b % 8).
__device__ __forceinline__ void tile_coords(int nb, int b, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  constexpr int GROUP_M = 4;
  const int L = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  const int per_group = GROUP_M * tiles_n;
  const int grp = L / per_group;
  const int first_m = grp * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in = L % per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

// Upper-triangle tiles of a T x T tile grid (symmetric products): block b -> the b-th tile
// (tm <= tn) in row order.
__device__ __forceinline__ void tri_coords(int T, int& tm, int& tn) {
  int L = blockIdx.x, r = 0;
  while (L >= T - r) {
    L -= T - r;
    ++r;
  }
  tm = r;
  tn = r + L;
}

// Register-staged kernel, launched for fp32 operands (the parity configurations) with 64 x 64
// tiles: BM x BN output tile per workgroup, each wave computing (BM/2) x (BN/2) as (BM/64) x
// (BN/64) MFMA tiles of 32 x 32 (v_mfma_f32_32x32x2f32, eight per 16-wide K slice); operand
// tiles go global -> registers -> LDS (padded rows; RC operands transposed in registers), the
// next K tile loaded into registers while the current one is multiplied.
template <typename T, int BM, int BN, bool A_KC, bool B_KC, class Epi, int SITE>
__global__ __launch_bounds__(THREADS, (BM * BN >= 256 * 256) ? 1 : 2) void gemm_kernel(
    const T* __restrict__ A, long long lda, const T* __restrict__ B, long long ldb, int M, int N,
    int K, uint32_t a_bytes, uint32_t b_bytes, Epi epi) {
  using C = Cfg<T>;
  constexpr int TM = BM / 64, TN = BN / 64;  // MFMA tiles per wave
  __shared__ __attribute__((aligned(16))) T lds[2][(BM + BN) * C::PITCH];
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(gridDim.x, blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
  const int wm = (w / 2) * (BM / 2), wn = (w % 2) * (BN / 2);
  const int lr = lane % 32, lg = lane / 32;

  Stage<T, BM, A_KC> sa;
  Stage<T, BN, B_KC> sb;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, a_bytes), rb = make_rsrc(B, b_bytes);
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int nk = (K + C::BK - 1) / C::BK;
  sa.load(ra, lda, m0, 0, M, K);
  sb.load(rb, ldb, n0, 0, N, K);
  sa.store(lds[0]);
  sb.store(lds[0] + BM * C::PITCH);
  sa.load(ra, lda, m0, C::BK, M, K);  // loads past K are predicated off (zeros)
  sb.load(rb, ldb, n0, C::BK, N, K);
  __syncthreads();

  // One barrier per K tile.  Each iteration first writes tile kt+1 (loaded one iteration ago)
  // into the idle buffer `cur ^ 1` and issues the loads of tile kt+2, then multiplies buffer
  // `cur`: global latency is hidden behind a full tile of MFMAs.  The scheduling fence keeps
  // the loads from sinking to the end of the loop.  On the last tiles the stores write unused
  // data and the loads are predicated off.
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    sa.store(lds[cur ^ 1]);
    sb.store(lds[cur ^ 1] + BM * C::PITCH);
    sa.load(ra, lda, m0, (kt + 2) * C::BK, M, K);
    sb.load(rb, ldb, n0, (kt + 2) * C::BK, N, K);
    __builtin_amdgcn_sched_barrier(0);
    const T* As = lds[cur];
    const T* Bs = lds[cur] + BM * C::PITCH;
    // fragments of the next 16-wide K slice are read while the current slice's MFMAs run
    vec8_t<T> af[2][TM], bfr[2][TN];
    auto read = [&](int ks, int slot) {
#pragma unroll
      for (int i = 0; i < TM; ++i) af[slot][i] = load8(As + (wm + i * 32 + lr) * C::PITCH + ks + lg * 8);
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[slot][j] = load8(Bs + (wn + j * 32 + lr) * C::PITCH + ks + lg * 8);
    };
    read(0, 0);
#pragma unroll
    for (int ks = 0; ks < C::BK; ks += 16) {
      const int slot = (ks / 16) & 1;
      if (ks + 16 < C::BK) read(ks + 16, slot ^ 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) Mma<T>::run(acc[i][j], bfr[slot][j], af[slot][i]);
    }
    __syncthreads();
  }

  // Epilogue through LDS (free once the last K tile is consumed).  The MFMA computed each
  // 32 x 32 tile transposed (B fragment first), so lane l holds output row l%32 and, in
  // registers 4q..4q+3, columns q*8 + (l/32)*4 + 0..3.  Each wave writes 32-row slices of its
  // (BM/2) x (BN/2) tile to its own LDS region (row pitch BN/2 + 4 floats: conflict-free), then
  // reads them back row-major so that 32 lanes cover 128 consecutive columns of one row: the
  // epilogue's global accesses are contiguous 256 B (bf16) / 512 B (fp32) row segments.
  {
    constexpr int WC = BN / 2, EP = WC + 4;  // wave tile columns, LDS row pitch in floats
    static_assert(4 * 32 * EP * 4 <= 2 * (BM + BN) * Cfg<T>::PITCH * (int)sizeof(T),
                  "epilogue staging must fit the operand buffers");
    float* ep = reinterpret_cast<float*>(&lds[0][0]) + w * 32 * EP;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {acc[i][j][q * 4], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2],
                           acc[i][j][q * 4 + 3]};
          *reinterpret_cast<f32x4*>(ep + lr * EP + j * 32 + q * 8 + lg * 4) = v;
        }
      // lanes 0..WC/4-1 take consecutive 4-column groups of one row; WAVE*4/WC rows per pass
      constexpr int LPR = WC / 4, RPP = WAVE / LPR;
#pragma unroll
      for (int rr = 0; rr < 32; rr += RPP) {
        const int r = rr + lane / LPR, c4 = (lane % LPR) * 4;
        const f32x4 x = *reinterpret_cast<const f32x4*>(ep + r * EP + c4);
        const int row = m0 + wm + i * 32 + r, col = n0 + wn + c4;
        if (row < M && col < N) {
          const float v[4] = {x[0], x[1], x[2], x[3]};
          epi(row, col, v);
        }
      }
    }
  }
}

// Epilogues with an at_batch(z) member serve batched launches.
template <class E, class = void>
struct has_batch : std::false_type {};
template <class E>
struct has_batch<E, std::void_t<decltype(std::declval<E&>().at_batch(0))>> : std::true_type {};

// ---------------------------------------------------------------- bf16: DMA-staged kernel
// Operand tiles travel global -> LDS by buffer loads that write LDS directly (16 B per lane,
// 1 KB per wave instruction, lane l to byte 16*l of the instruction's LDS block), in the
// operand's own global layout, so no staging registers and no LDS store instructions are used:
//  * K-contiguous tile: [ROWS][BK] bf16; 16 B chunk c of row r at chunk position c ^ kswz(r),
//    so that the 16 lanes of a fragment read that the LDS serves together hit 16 distinct
//    16-byte bank groups (64 banks of 4 bytes);
//  * row-contiguous tile: [BK k][ROWS] bf16, chunk c of k-row k at c ^ (4 * (k % 4)); its MFMA
//    fragments come from two transposing LDS reads (ds_read_b64_tr_b16: within a 16-lane
//    group, lane j receives element j%4 of lanes j/4 + 4i, i = 0..3; lane 4i + t addresses
//    row k0 + i, columns n0 + 4t .. +3, so lane j gets B[k0 .. k0+3][n0 + j]).
// Loads past the operand's end read as zeros (buffer range check).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(3))) float lds_f32;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4;

template <int ROWS, int BK, bool KC, int NW>
struct DmaTile {
  static_assert(BK == 32 || BK == 64, "K tile of 32 or 64");
  static constexpr int BYTES = ROWS * BK * 2;
  static constexpr int NI = BYTES / 1024 / NW;          // DMA instructions per wave (NW waves)
  static_assert(NI * NW * 1024 == BYTES, "tile must split evenly over the waves");
  static constexpr int CPR = BK / 8, RPI = 64 / CPR;   // KC: chunks per row, rows per instruction
  static __device__ __forceinline__ int kswz(int r) { return BK == 64 ? (r >> 1) & 7 : (r >> 2) & 3; }
  // issue this wave's DMA instructions for the tile at (row0, k0)
  static __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, long long ld, int row0,
                                               int k0, int rows_lim, int k_lim, bf16* tile) {
    const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = w * NI + i;  // 1 KB block of the tile
      uint32_t off;
      if constexpr (KC) {
        const int r = blk * RPI + lane / CPR, c = (lane % CPR) ^ kswz(r);
        const int row = row0 + r, k = k0 + c * 8;
        off = (row < rows_lim && k < k_lim) ? (uint32_t)(((long long)row * ld + k) * 2) : OOB;
      } else {
        constexpr int CPK = ROWS / 8, KPI = 1024 / (ROWS * 2);  // chunks per k-row, k-rows per block
        const int kk = blk * KPI + lane / CPK, c = (lane % CPK) ^ (4 * (kk % 4));
        const int row = row0 + c * 8, k = k0 + kk;
        off = (row < rows_lim && k < k_lim) ? (uint32_t)(((long long)k * ld + row) * 2) : OOB;
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(tile + blk * 512), 16, off, 0, 0, 0);
    }
  }
  // 8 consecutive K values (k = ks + g*8 .. +7) of tile row r (r = lane's row)
  static __device__ __forceinline__ bf16x8 frag(const bf16* tile, int r, int ks, int lane) {
    const int g = (lane / 32) % 2;
    if constexpr (KC) {
      const int c = ks / 8 + g;
      return load8(tile + r * BK + ((c ^ kswz(r)) * 8));
    } else {
      // r = rowbase + lane % 32; the 16-lane group of this lane covers rows nb .. nb+15
      const int j = lane % 16, i = j / 4, t = j % 4;
      const int nb = r - j;
      bf16x8 v;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = ks + g * 8 + h * 4 + i;
        const int n = nb + 4 * t;
        const int pos = (((n / 8) ^ (4 * (k % 4))) * 8) + (n % 8);
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(tile + k * ROWS + pos));
        const bf16x4 y = __builtin_bit_cast(bf16x4, x);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[h * 4 + e] = y[e];
      }
      return v;
    }
  }
};

// f(integral_constant<int, 0>) ... f(integral_constant<int, N - 1>), unrolled
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>());
}

// Stage S of a kernel's LDS ring: an array of its own, so the compiler can tell the LDS reads of
// one stage from DMA writes still in flight into another (reads of an array that a DMA may be
// writing make it wait for all outstanding DMA).
template <int S, int BYTES>
__device__ __forceinline__ bf16* lds_stage() {
  __shared__ __attribute__((aligned(1024))) bf16 buf[BYTES / 2];
  return buf;
}
// Wait until at most N vector-memory operations of this wave are outstanding and all its LDS
// operations are done (s_waitcnt fields: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | ((N >> 4) << 14));
}

// BM x BN tile per workgroup of WGM x WGN waves; each wave computes (BM/WGM) x (BN/WGN) as
// 32 x 32 MFMA tiles.  K advances in BK-wide tiles through a ring of NS LDS stages: the DMA of
// tile kt + NS - 1 is issued while tile kt is multiplied, so NS - 1 tiles of loads are in flight
// behind the MFMAs.  One barrier per K tile (after this wave's DMA of tile kt has landed, so all
// waves' have; the stage read in the previous iteration is then free for the next DMA).  The
// 256 x 256 tile runs 8 waves, two per SIMD; the 128 x 128 tile 4 waves, two workgroups per CU.
// The workgroup computes tile `vb` of the `nvb` tiles of its problem (blockIdx.x and gridDim.x
// for a plain launch).
template <int BM, int BN, int WGM, int WGN, int BK, int NS, bool A_KC, bool B_KC, class Epi>
__device__ __forceinline__ void gemm_dma_tile(
    const bf16* A, long long lda, const bf16* B, long long ldb, int M,
    int N, int K, uint32_t a_bytes, uint32_t b_bytes, Epi epi, int kps, long long a_bs,
    long long b_bs, int vb, int nvb) {
  constexpr int NW = WGM * WGN, WTM = BM / WGM, WTN = BN / WGN;
  // batch z = blockIdx.z: operands at A + z * a_bs, B + z * b_bs; epilogues that hold batched
  // outputs move their pointers themselves
  A += (long long)blockIdx.z * a_bs;
  B += (long long)blockIdx.z * b_bs;
  if constexpr (has_batch<Epi>::value) epi.at_batch(blockIdx.z);
  // split-K: workgroups with blockIdx.y = s take K range [s * kps, min(K, (s + 1) * kps))
  {
    const int k0 = blockIdx.y * kps;
    A += A_KC ? (long long)k0 : (long long)k0 * lda;
    B += B_KC ? (long long)k0 : (long long)k0 * ldb;
    K = min(K - k0, kps);
  }
  constexpr int TM = WTM / 32, TN = WTN / 32;
  using TA = DmaTile<BM, BK, A_KC, NW>;
  using TB = DmaTile<BN, BK, B_KC, NW>;
  constexpr int PER_TILE = TA::NI + TB::NI;  // DMA instructions per wave per K tile
  static_assert(NS >= 2 && (NS - 2) * PER_TILE < 64, "pipeline depth");
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  if constexpr (is_symmetric<Epi>::value) tri_coords(tiles_m, tm, tn);
  else tile_coords(nvb, vb, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
  const int wm = (w / WGN) * WTM, wn = (w % WGN) * WTN;
  const int lr = lane % 32, lg = lane / 32;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, a_bytes), rb = make_rsrc(B, b_bytes);
  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  const int nk = (K + BK - 1) / BK;
  // DMA of K tile kt into stage S (branch-free: tiles past K read zeros and are never used)
  auto issue = [&](auto s_c, int kt) {
    TA::issue(ra, lda, m0, kt * BK, M, K, lds_stage<decltype(s_c)::value, BM * BK * 2>());
    TB::issue(rb, ldb, n0, kt * BK, N, K, lds_stage<NS + decltype(s_c)::value, BN * BK * 2>());
  };
  // Fragments: slot 0 holds the first 16-wide K slice of the current tile, read during the
  // previous tile's last MFMAs (so the barrier between tiles costs no LDS latency); each slice's
  // successor is read while its MFMAs run.
  bf16x8 af[2][TM], bfr[2][TN];
  auto read = [&](const bf16* As, const bf16* Bs, int ks, int slot) {
#pragma unroll
    for (int i = 0; i < TM; ++i) af[slot][i] = TA::frag(As, wm + i * 32 + lr, ks, lane);
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[slot][j] = TB::frag(Bs, wn + j * 32 + lr, ks, lane);
  };
  auto stage_a = [&](auto s_c) -> const bf16* {
    return lds_stage<decltype(s_c)::value, BM * BK * 2>();
  };
  auto stage_b = [&](auto s_c) -> const bf16* {
    return lds_stage<NS + decltype(s_c)::value, BN * BK * 2>();
  };
  // MFMAs of the tile in stage S, then slice 0 of the tile in stage S + 1
  auto compute = [&](auto s_c) {
    using SN = std::integral_constant<int, (decltype(s_c)::value + 1) % NS>;
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      const int slot = (ks / 16) & 1;
      if (ks + 16 < BK) read(stage_a(s_c), stage_b(s_c), ks + 16, slot ^ 1);
      else read(stage_a(SN()), stage_b(SN()), 0, slot ^ 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) Mma<bf16>::run(acc[i][j], bfr[slot][j], af[slot][i]);
    }
  };
  static_assert(BK % 32 == 0, "slot 0 must hold the first slice of every tile");
  constexpr int NSL = BK / 16;  // 16-wide K slices per tile
  if constexpr (NS >= 3) {
    // iteration kt, on stage S = kt % NS: the barrier comes first, then the DMA of tile
    // kt + NS - 1 into the stage freed by the previous iteration
    auto step = [&](auto s_c, int kt) {
      constexpr int S = decltype(s_c)::value;
      wait_vm_lds<(NS - 3) * PER_TILE>();  // this wave's DMA of tile kt + 1 has landed
      __builtin_amdgcn_s_barrier();         // ... and every wave's; stage S - 1 is free
      __builtin_amdgcn_sched_barrier(0);
      issue(std::integral_constant<int, (S + NS - 1) % NS>(), kt + NS - 1);
      if (kt < nk) compute(s_c);
      // keep the next iteration's wait and barrier behind these MFMAs
      __builtin_amdgcn_sched_barrier(0);
    };
    static_for<NS - 1>([&](auto s_c) { issue(s_c, decltype(s_c)::value); });
    wait_vm_lds<(NS - 2) * PER_TILE>();  // tile 0
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read(stage_a(std::integral_constant<int, 0>()), stage_b(std::integral_constant<int, 0>()), 0, 0);
    for (int kt = 0; kt < nk; kt += NS)
      static_for<NS>([&](auto s_c) { step(s_c, kt + decltype(s_c)::value); });
  } else {
    // two stages (64-wide K tiles, so K-contiguous rows are whole 128-byte lines): iteration kt
    // issues the DMA of tile kt + 1 into the other stage (every wave has read all of tile kt - 1
    // before the previous barrier), multiplies slices 0 .. NSL-2, waits for that DMA and meets
    // the other waves at the barrier, then multiplies the last slice while reading the first
    // slice of tile kt + 1
    static_assert(NS == 2, "two or at least three stages");
    auto step = [&](auto s_c, int kt) {
      constexpr int S = decltype(s_c)::value;
      using SN = std::integral_constant<int, S ^ 1>;
      issue(SN(), kt + 1);
      __builtin_amdgcn_sched_barrier(0);
      if (kt < nk) {
#pragma unroll
        for (int sl = 0; sl < NSL - 1; ++sl) {
          const int slot = sl & 1;
          if (sl + 1 < NSL - 1) read(stage_a(s_c), stage_b(s_c), (sl + 1) * 16, slot ^ 1);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) Mma<bf16>::run(acc[i][j], bfr[slot][j], af[slot][i]);
        }
        // the last slice's fragments, then the barrier (the reads have completed by then)
        read(stage_a(s_c), stage_b(s_c), (NSL - 1) * 16, (NSL - 1) & 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      wait_vm_lds<0>();               // this wave's DMA of tile kt + 1 has landed
      __builtin_amdgcn_s_barrier();   // ... and every wave's; all reads of tile kt are done
      __builtin_amdgcn_sched_barrier(0);
      if (kt < nk) {
        constexpr int slot = (NSL - 1) & 1;
        read(stage_a(SN()), stage_b(SN()), 0, slot ^ 1);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) Mma<bf16>::run(acc[i][j], bfr[slot][j], af[slot][i]);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    issue(std::integral_constant<int, 0>(), 0);
    wait_vm_lds<0>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    read(stage_a(std::integral_constant<int, 0>()), stage_b(std::integral_constant<int, 0>()), 0, 0);
    for (int kt = 0; kt < nk; kt += 2) {
      step(std::integral_constant<int, 0>(), kt);
      step(std::integral_constant<int, 1>(), kt + 1);
    }
  }
  // drain the DMA of the tiles past K before the epilogue reuses the stages
  wait_vm_lds<0>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);

  // Epilogue through LDS.  The MFMA computed each 32 x 32 tile transposed (B fragment first), so
  // lane l holds output row l%32 and, in registers 4q..4q+3, columns q*8 + (l/32)*4 + 0..3.  Each
  // wave writes 32-row slices of its tile to its own LDS region (32 rows x WTN floats, 16-byte
  // chunk c of row r at chunk c ^ (r % 16): conflict-free for the column writes and the row
  // reads), then reads them back row-major so that consecutive lanes cover consecutive 4-column
  // groups of one row.  The regions lie in the A halves of the stages.
  static_assert(WTN % 64 == 0, "epilogue staging assumes wave tiles of 64-column multiples");
  constexpr int REGION = 32 * WTN * 4;
  constexpr int WPA = BM * BK * 2 / REGION, WPB = BN * BK * 2 / REGION;  // regions per half
  static_assert(NS * (WPA + WPB) >= NW, "epilogue staging must fit the stages");
  // loads of at most PG passes are in flight together (all of a slice's unless the epilogue
  // limits it, for the registers its loads take)
  constexpr int LPR = WTN / 4, RPP = WAVE / LPR, NP = 32 / RPP;
  constexpr int PG = epi_pass_group<Epi>() < NP ? epi_pass_group<Epi>() : NP;
  static_assert(NP % PG == 0, "pass groups divide the slice");
  auto epilogue = [&](lds_f32* ep) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 v = {acc[i][j][q * 4], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2],
                           acc[i][j][q * 4 + 3]};
          const int chunk = (j * 32 + q * 8 + lg * 4) / 4;
          *reinterpret_cast<lds_f32x4*>(ep + lr * WTN + ((chunk ^ (lr % 16)) * 4)) = v;
        }
      if constexpr (epi_pairs<Epi>::value) {
        // rotation-pair epilogues: each lane takes four pairs of one row (columns c..c+3 and
        // c+hd/2..c+hd/2+3 of a head), WTN/8 lanes per row; loads of a whole slice first
        constexpr int LP2 = WTN / 8, RP2 = WAVE / LP2, NP2 = 32 / RP2;
        const int hd = epi.hd, jl = lane % LP2, hq = hd / 8;
        const int cw = (jl / hq) * hd + (jl % hq) * 4;  // column inside the wave tile
        const int colp = n0 + wn + cw;
        typename Epi::Pre pre[NP2];
#pragma unroll
        for (int p = 0; p < NP2; ++p) {
          const int row = m0 + wm + i * 32 + p * RP2 + lane / LP2;
          pre[p] = epi.load(min(row, M - 1), colp);
        }
#pragma unroll
        for (int p = 0; p < NP2; ++p) {
          const int r = p * RP2 + lane / LP2;
          const f32x4 a = *reinterpret_cast<const lds_f32x4*>(ep + r * WTN + (((cw / 4) ^ (r % 16)) * 4));
          const int cw2 = cw + hd / 2;
          const f32x4 b = *reinterpret_cast<const lds_f32x4*>(ep + r * WTN + (((cw2 / 4) ^ (r % 16)) * 4));
          const int row = m0 + wm + i * 32 + r;
          if (row < M) {
            const float x1[4] = {a[0], a[1], a[2], a[3]}, x2[4] = {b[0], b[1], b[2], b[3]};
            epi.store(row, colp, x1, x2, pre[p]);
          }
        }
      } else {
        // each group's epilogue loads first (at in-range addresses, no per-lane branches), then
        // its stores
        const int c4 = (lane % LPR) * 4, col = n0 + wn + c4;
#pragma unroll
        for (int p0 = 0; p0 < NP; p0 += PG) {
          typename Epi::Pre pre[PG];
#pragma unroll
          for (int p = 0; p < PG; ++p) {
            const int row = m0 + wm + i * 32 + (p0 + p) * RPP + lane / LPR;
            pre[p] = epi.load(min(row, M - 1), min(col, N - 4));
          }
#pragma unroll
          for (int p = 0; p < PG; ++p) {
            const int r = (p0 + p) * RPP + lane / LPR;
            const f32x4 x = *reinterpret_cast<const lds_f32x4*>(ep + r * WTN + (((c4 / 4) ^ (r % 16)) * 4));
            const int row = m0 + wm + i * 32 + r;
            if (row < M && col < N) {
              const float v[4] = {x[0], x[1], x[2], x[3]};
              epi.store(row, col, v, pre[p]);
            }
          }
        }
      }
      if constexpr (is_symmetric<Epi>::value) {
        // off-diagonal tiles of a symmetric product: lane c reads column c of the staged 32-row
        // slice and writes it as the run out[n0 + wn + c][m0 + wm + i*32 ..] (tile-aligned sizes)
        static_assert(WTN == WAVE, "the column read-back gives each lane one column");
        if (tm != tn) {
          const int c = lane, r0 = m0 + wm + i * 32;
          float cv[32];
#pragma unroll
          for (int r = 0; r < 32; ++r) cv[r] = ep[r * WTN + (((c / 4) ^ (r % 16)) * 4) + c % 4];
          epi.mirror_col(r0, n0 + wn + c, cv);
        }
      }
    }
  };
  // Wave w stages through region w of the stages' A halves, then of their B halves.  The region
  // pointer stays in the LDS address space (a generic pointer would turn the accesses into flat
  // ones, which wait on global memory traffic too).
  lds_f32* halves[2 * NS];
  static_for<NS>([&](auto s_c) {
    halves[decltype(s_c)::value] = (lds_f32*)lds_stage<decltype(s_c)::value, BM * BK * 2>();
    halves[NS + decltype(s_c)::value] = (lds_f32*)lds_stage<NS + decltype(s_c)::value, BN * BK * 2>();
  });
  if (w < NS * WPA) epilogue(halves[w / WPA] + (w % WPA) * (REGION / 4));
  else epilogue(halves[NS + (w - NS * WPA) / WPB] + ((w - NS * WPA) % WPB) * (REGION / 4));
}

template <int BM, int BN, int WGM, int WGN, int BK, int NS, bool A_KC, bool B_KC, class Epi,
          int SITE>
__global__ __launch_bounds__(64 * WGM * WGN, (BM * BN >= 256 * 256) ? 1 : 2) void gemm_dma_kernel(
    const bf16* A, long long lda, const bf16* B, long long ldb, int M,
    int N, int K, uint32_t a_bytes, uint32_t b_bytes, Epi epi, int kps, long long a_bs,
    long long b_bs) {
  gemm_dma_tile<BM, BN, WGM, WGN, BK, NS, A_KC, B_KC, Epi>(A, lda, B, ldb, M, N, K, a_bytes,
                                                           b_bytes, epi, kps, a_bs, b_bs,
                                                           blockIdx.x, gridDim.x);
}

// One operand pair of a paired launch (the same layouts, tile size and epilogue type).
template <class Epi>
struct GemmProb {
  const bf16 *A, *B;
  long long lda, ldb;
  int M, N, K;
  uint32_t a_bytes, b_bytes;
  Epi epi;
  int tiles;
};
// Two independent products in one launch: blocks 0 .. p0.tiles-1 compute p0's tiles, the rest
// p1's (each walked in its own XCD-grouped order), so that two products that would each leave
// CUs idle fill one round of the chip together.
template <int BM, int BN, int WGM, int WGN, int BK, int NS, bool A_KC, bool B_KC, class Epi,
          int SITE>
__global__ __launch_bounds__(64 * WGM * WGN, (BM * BN >= 256 * 256) ? 1 : 2) void gemm_dma_pair_kernel(
    GemmProb<Epi> p0, GemmProb<Epi> p1) {
  const bool second = (int)blockIdx.x >= p0.tiles;
  const GemmProb<Epi>& p = second ? p1 : p0;
  gemm_dma_tile<BM, BN, WGM, WGN, BK, NS, A_KC, B_KC, Epi>(
      p.A, p.lda, p.B, p.ldb, p.M, p.N, p.K, p.a_bytes, p.b_bytes, p.epi, p.K, 0, 0,
      (int)blockIdx.x - (second ? p0.tiles : 0), p.tiles);
}

// Calls f with an epilogue whose loads do not depend on run-time flags: accumulate vs overwrite
// and present vs absent addends become distinct types (a load that a flag may skip leaves the
// kernel unable to count its outstanding loads, so it waits for all of them).
template <class Epi, class F>
inline void with_static_epi(const Epi& e, F&& f) { f(e); }
template <class F>
inline void with_static_epi(const EpiStoreF32& e, F&& f) {
  if (e.beta) f(EpiAccF32{e.out, e.ldo});
  else f(EpiPutF32{e.out, e.ldo});
}
template <typename T, class F>
inline void with_static_epi(const EpiQKV<T>& e, F&& f) {
  if (e.u) f(e);
  else f(EpiStore<T>{e.out, e.ldo});
}
template <typename T, class F>
inline void with_static_epi(const EpiAddRows<T>& e, F&& f) {
  if (e.add) f(e);
  else f(EpiPutF32{e.out, e.ld});
}

// Bytes spanned by an operand of `rows` x K (KC: rows of ld; RC: K rows of ld).
inline long long operand_bytes(bool kc, long long rows, long long K, long long ld, long long es) {
  return (kc ? (rows - 1) * ld + K : (K - 1) * ld + rows) * es;
}

// Compute units of the current device (cached per device; 256 if the query fails).
inline unsigned resident_cus() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cached[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    cached[dev] = cus;
  }
  return (unsigned)cached[dev];
}

template <int BM, int BN, int WGM, int WGN, class Epi, int SITE>
void launch_dma(bool a_kc, bool b_kc, int M, int N, int K, const bf16* A, long long lda,
                const bf16* B, long long ldb, const Epi& epi, hipStream_t s, int splits = 1,
                int batch = 1, long long a_bs = 0, long long b_bs = 0) {
  const int kps = splits > 1 ? (int)cdiv(cdiv(K, splits), 64) * 64 : K;  // K per split
  const long long T = cdiv(M, BM);  // symmetric products: the upper triangle of a T x T grid
  const long long tiles = is_symmetric<Epi>::value ? T * (T + 1) / 2 : (long long)cdiv(M, BM) * cdiv(N, BN);
  dim3 grid((unsigned)tiles, (unsigned)cdiv(K, kps), (unsigned)batch);
  // each split's operand spans at most these bytes from its own start
  const uint32_t ab = (uint32_t)operand_bytes(a_kc, M, kps, lda, 2);
  const uint32_t bb = (uint32_t)operand_bytes(b_kc, N, kps, ldb, 2);
  // A K-contiguous A reads whole 128-byte lines only with 64-wide K tiles, which leave room for
  // two stages; with a row-contiguous A (whole lines at any depth) four 32-wide stages are used
  // (the 64-wide two-stage form of that layout does not fit the registers)
#define GEMM_DMA(AK, BK_, KT, NS_)                                                               \
  gemm_dma_kernel<BM, BN, WGM, WGN, KT, NS_, AK, BK_, Epi, SITE><<<grid, 64 * WGM * WGN, 0, s>>>( \
      A, lda, B, ldb, M, N, K, ab, bb, epi, kps, a_bs, b_bs)
  if constexpr (epi_wave_cols<Epi>::value != 64) {
    // epilogues with wide wave tiles serve forward projections (both operands K-contiguous;
    // gemm() rejects the other layouts for them)
    GEMM_DMA(true, true, 64, 2);
  } else {
    if (a_kc && b_kc) GEMM_DMA(true, true, 64, 2);
    else if (a_kc) GEMM_DMA(true, false, 64, 2);
    else if (b_kc) GEMM_DMA(false, true, 32, 4);
    else GEMM_DMA(false, false, 32, 4);
  }
#undef GEMM_DMA
}

template <typename T, int BM, int BN, class Epi, int SITE>
void launch_tiles(bool a_kc, bool b_kc, int M, int N, int K, const T* A, long long lda,
                  const T* B, long long ldb, const Epi& epi, hipStream_t s) {
  dim3 grid((unsigned)(cdiv(M, BM) * cdiv(N, BN)));
  const uint32_t ab = (uint32_t)operand_bytes(a_kc, M, K, lda, sizeof(T));
  const uint32_t bb = (uint32_t)operand_bytes(b_kc, N, K, ldb, sizeof(T));
#define GEMM_GO(AK, BK_)                                                                        \
  gemm_kernel<T, BM, BN, AK, BK_, Epi, SITE><<<grid, THREADS, 0, s>>>(A, lda, B, ldb, M, N, K, ab, \
                                                                     bb, epi)
  if (a_kc && b_kc) GEMM_GO(true, true);
  else if (a_kc) GEMM_GO(true, false);
  else if (b_kc) GEMM_GO(false, true);
  else GEMM_GO(false, false);
#undef GEMM_GO
}

}  // namespace gemm_detail

namespace gemm_detail {
// Tile size of a bf16 product from the quantisation of its output tiling.  A 256 x 256 tile
// (one workgroup per CU) does about 1.25x the work per CU-cycle of two co-resident 128 x 128
// tiles (measured at K = 768 and 2048), but with 256 tiles per round a last, partly filled round
// can leave most CUs idle (GPT-2-small's 8192 x 2304 q/k/v projection: 288 tiles, two rounds,
// 56% busy; as 128 x 128 tiles, 1152 over 512 slots, 75%).  Whichever tiling keeps more of the
// chip's slots busy, weighted by that factor, is used; a product whose 128 x 128 tiles each get
// a CU of their own takes them (a quarter of the work per CU, no round to fill).
inline bool prefer_big_tiles(long long tiles256, long long tiles128) {
  if (tiles128 <= 256) return false;
  auto busy = [](long long t, long long slots) {
    return (double)t / (double)(slots * ((t + slots - 1) / slots));
  };
  return 1.25 * busy(tiles256, 256) >= busy(tiles128, 512);
}
}  // namespace gemm_detail

// C[m,n] = sum_k A(m,k) B(n,k); a_kc/b_kc select K-contiguous (p[r*ld+k]) or row-contiguous
// (p[k*ld+r]) operands.  Requirements: K % 8 == 0, lda/ldb % 8 == 0, 16-byte aligned operands,
// M % 8 == 0 for a row-contiguous A, N % 8 == 0 for a row-contiguous B, N % 4 == 0 and output
// leading dimensions (inside the epilogue) multiples of 4.  bf16 problems use 256 x 256 or
// 128 x 128 tiles as prefer_big_tiles decides; fp32 uses 64 x 64.
template <int SITE, typename T, class Epi>
inline gpt_status gemm(bool a_kc, bool b_kc, int M, int N, int K, const T* A, long long lda,
                       const T* B, long long ldb, const Epi& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return GPT_OK;
  if (K <= 0 || K % 8) return fail(GPT_ESHAPE, "gemm: K must be a positive multiple of 8");
  if (lda % 8 || ldb % 8) return fail(GPT_ESHAPE, "gemm: leading dimensions must be multiples of 8");
  if ((!a_kc && M % 8) || (!b_kc && N % 8))
    return fail(GPT_ESHAPE, "gemm: row-contiguous operands need a multiple of 8 rows");
  if (N % 4) return fail(GPT_ESHAPE, "gemm: N must be a multiple of 4");
  if (((uintptr_t)A | (uintptr_t)B) % 16) return fail(GPT_EINVAL, "gemm: operands must be 16-byte aligned");
  if (gemm_detail::operand_bytes(a_kc, M, K, lda, sizeof(T)) > (1LL << 31) ||
      gemm_detail::operand_bytes(b_kc, N, K, ldb, sizeof(T)) > (1LL << 31))
    return fail(GPT_ESHAPE, "gemm: each operand must span at most 2 GiB");
  if (epi_wave_cols<Epi>::value != 64 && (!a_kc || !b_kc || !std::is_same<T, bf16>::value))
    return fail(GPT_EINVAL, "gemm: this epilogue needs bf16 K-contiguous operands");
  if ((long long)cdiv(M, 128) * cdiv(N, 128) >= (1LL << 31)) return fail(GPT_ESHAPE, "gemm: too many tiles");
  const bool big = gemm_detail::prefer_big_tiles((long long)cdiv(M, 256) * cdiv(N, 256),
                                                 (long long)cdiv(M, 128) * cdiv(N, 128));
  gemm_detail::with_static_epi(epi, [&](const auto& e) {
    using E = typename std::decay<decltype(e)>::type;
    if constexpr (std::is_same<T, bf16>::value) {
      if constexpr (epi_wave_cols<E>::value == 128) {
        // wave tiles of 64 x 128 (4 x 2 waves) or 32 x 128 (4 x 1)
        if (big)
          gemm_detail::launch_dma<256, 256, 4, 2, E, SITE>(a_kc, b_kc, M, N, K, A, lda, B, ldb, e, s);
        else
          gemm_detail::launch_dma<128, 128, 4, 1, E, SITE>(a_kc, b_kc, M, N, K, A, lda, B, ldb, e, s);
      } else if (big) {
        gemm_detail::launch_dma<256, 256, 2, 4, E, SITE>(a_kc, b_kc, M, N, K, A, lda, B, ldb, e, s);
      } else {
        gemm_detail::launch_dma<128, 128, 2, 2, E, SITE>(a_kc, b_kc, M, N, K, A, lda, B, ldb, e, s);
      }
    } else {
      // fp32 serves the small parity configurations only
      gemm_detail::launch_tiles<T, 64, 64, E, SITE>(a_kc, b_kc, M, N, K, A, lda, B, ldb, e, s);
    }
  });
  return check_launch("gemm");
}

// Batched bf16 GEMM: C_z = A_z B_z^T for z < batch, with A_z = A + z * a_bs and B_z = B + z * b_bs
// (elements) in the layouts of gemm(), and an epilogue whose at_batch(z) moves its outputs.  The
// tile size follows the total tile count over the batch.
template <int SITE, class Epi>
inline gpt_status gemm_batched(bool a_kc, bool b_kc, int M, int N, int K, const bf16* A,
                               long long lda, long long a_bs, const bf16* B, long long ldb,
                               long long b_bs, int batch, const Epi& epi, hipStream_t s) {
  static_assert(gemm_detail::has_batch<Epi>::value, "batched launches need an at_batch epilogue");
  if (batch <= 0 || M <= 0 || N <= 0) return GPT_OK;
  if (is_symmetric<Epi>::value && (M != N || M % 256))
    return fail(GPT_ESHAPE, "gemm_batched: a symmetric product is square with a multiple of 256 rows");
  if (batch > 65535) return fail(GPT_ESHAPE, "gemm_batched: at most 65535 matrices");
  if (K <= 0 || K % 8) return fail(GPT_ESHAPE, "gemm: K must be a positive multiple of 8");
  if (lda % 8 || ldb % 8 || a_bs % 8 || b_bs % 8)
    return fail(GPT_ESHAPE, "gemm_batched: leading dimensions and batch strides must be multiples of 8");
  if ((!a_kc && M % 8) || (!b_kc && N % 8))
    return fail(GPT_ESHAPE, "gemm: row-contiguous operands need a multiple of 8 rows");
  if (N % 4) return fail(GPT_ESHAPE, "gemm: N must be a multiple of 4");
  if (((uintptr_t)A | (uintptr_t)B) % 16) return fail(GPT_EINVAL, "gemm: operands must be 16-byte aligned");
  if (gemm_detail::operand_bytes(a_kc, M, K, lda, 2) > (1LL << 31) ||
      gemm_detail::operand_bytes(b_kc, N, K, ldb, 2) > (1LL << 31))
    return fail(GPT_ESHAPE, "gemm: each operand must span at most 2 GiB");
  if ((long long)cdiv(M, 128) * cdiv(N, 128) >= (1LL << 31)) return fail(GPT_ESHAPE, "gemm: too many tiles");
  const long long big_tiles = (long long)cdiv(M, 256) * cdiv(N, 256) * batch;
  if (big_tiles >= 240)
    gemm_detail::launch_dma<256, 256, 2, 4, Epi, SITE>(a_kc, b_kc, M, N, K, A, lda, B, ldb, epi, s,
                                                       1, batch, a_bs, b_bs);
  else
    gemm_detail::launch_dma<128, 128, 2, 2, Epi, SITE>(a_kc, b_kc, M, N, K, A, lda, B, ldb, epi, s,
                                                       1, batch, a_bs, b_bs);
  return check_launch("gemm_batched");
}

namespace gemm_detail {

// Split-K for bf16 GEMMs with an fp32 output (weight gradients) whose output tiling alone leaves
// CUs idle.  The shapes of the shipped workloads take the plan measured best on MI355X (a sweep
// of tile size x 1..16 splits, GEMM plus reduction, same box); other shapes: 256 x 256 tiles with
// 2..8 splits of >= 1024 K each when that gives >= 480 workgroups (about two per CU), else
// 128 x 128 tiles (two workgroups per CU) with up to 16 splits of >= 512 K.  A function of the
// shape only, so workspace sizing and launch agree.
struct SplitPlan {
  int splits;
  bool big;
};
struct TunedSplit {
  int M, N, K;
  SplitPlan plan;
};
// (µs per product on the sweep's box: best plan vs the general rule's)
constexpr TunedSplit kTunedSplits[] = {
    // GPT-2-small weight gradients over 8,192 tokens (also the speedrun micro-batches)
    {3072, 768, 8192, {2, false}},   // MLP up:   61.7 vs 63.6-73.4 (128 x 128, 4 splits)
    {768, 3072, 8192, {2, false}},   // MLP down: 58.9 vs 63.0-63.7
    {2304, 768, 8192, {4, false}},   // q/k/v:    40.0 vs 50.9-51.0 (8 splits)
    {768, 768, 8192, {4, false}},    // out, trigram projection: 26.6 vs 39.9 (16 splits)
    // d32 weight gradients over 16,384 tokens
    {2048, 2048, 16384, {4, true}},  // out:   132-134 vs 160-162 (256 x 256, 8 splits)
    {6144, 2048, 16384, {1, true}},  // q/k/v: 350-354 vs 394-396 (256 x 256, 4 splits)
};
inline SplitPlan split_plan(int M, int N, int K) {
  for (const TunedSplit& t : kTunedSplits)
    if (t.M == M && t.N == N && t.K == K) return t.plan;
  const long long t256 = (long long)cdiv(M, 256) * cdiv(N, 256);
  if (t256 >= 240) return {1, true};
  for (int sp = 2; sp <= 8; sp *= 2)
    if (t256 * sp >= 480 && K / sp >= 1024) return {sp, true};
  const long long t128 = (long long)cdiv(M, 128) * cdiv(N, 128);
  int sp = 1;
  while (sp < 16 && t128 * sp < 512 && K / (2 * sp) >= 512) sp *= 2;
  return {sp, false};
}

// out[m][n] = (beta ? out[m][n] : 0) + sum over splits s (in order) of ws[s][m][n]; N % 4 == 0.
template <int UNUSED = 0>
__global__ void splitk_reduce_kernel(const float* __restrict__ ws, long long stride, int splits,
                                     float* __restrict__ out, long long ldo, int M, int N,
                                     int beta) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const int n4 = N / 4;
  if (i >= (long long)M * n4) return;
  const long long r = i / n4;
  const int c = (int)(i % n4) * 4;
  f32x4 acc = *reinterpret_cast<const f32x4*>(ws + r * N + c);
  for (int sp = 1; sp < splits; ++sp) acc += *reinterpret_cast<const f32x4*>(ws + sp * stride + r * N + c);
  f32x4* o = reinterpret_cast<f32x4*>(out + r * ldo + c);
  if (beta) acc = *o + acc;
  *o = acc;
}

}  // namespace gemm_detail

// fp32 workspace (elements) a gemm_wgrad of this shape needs.
inline long long gemm_wgrad_ws_floats(int M, int N, int K) {
  const gemm_detail::SplitPlan sp = gemm_detail::split_plan(M, N, K);
  return sp.splits > 1 ? (long long)sp.splits * M * N : 0;
}

// GEMM with an fp32 output (weight gradients, and the input gradients that feed the fp32
// residual stream; beta as in EpiStoreF32): bf16 shapes that leave CUs idle are split over K
// into fp32 partials in `ws` and reduced in split order (deterministic).
template <int SITE, typename T>
inline gpt_status gemm_wgrad(bool a_kc, bool b_kc, int M, int N, int K, const T* A, long long lda,
                             const T* B, long long ldb, const EpiStoreF32& epi, float* ws,
                             long long ws_floats, hipStream_t s) {
  if constexpr (!std::is_same<T, bf16>::value) {
    return gemm<SITE, T>(a_kc, b_kc, M, N, K, A, lda, B, ldb, epi, s);
  } else {
    const gemm_detail::SplitPlan sp = gemm_detail::split_plan(M, N, K);
    if (sp.splits == 1 || M <= 0 || N <= 0) return gemm<SITE, T>(a_kc, b_kc, M, N, K, A, lda, B, ldb, epi, s);
    if (!ws || ws_floats < (long long)sp.splits * M * N)
      return fail(GPT_EWORKSPACE, "gemm_wgrad: split-K workspace too small");
    // same argument checks as gemm()
    if (K <= 0 || K % 8) return fail(GPT_ESHAPE, "gemm: K must be a positive multiple of 8");
    if (lda % 8 || ldb % 8) return fail(GPT_ESHAPE, "gemm: leading dimensions must be multiples of 8");
    if ((!a_kc && M % 8) || (!b_kc && N % 8))
      return fail(GPT_ESHAPE, "gemm: row-contiguous operands need a multiple of 8 rows");
    if (N % 4 || epi.ldo % 4) return fail(GPT_ESHAPE, "gemm: N and ldo must be multiples of 4");
    if (((uintptr_t)A | (uintptr_t)B) % 16 || ((uintptr_t)ws | (uintptr_t)epi.out) % 16)
      return fail(GPT_EINVAL, "gemm: operands must be 16-byte aligned");
    if (gemm_detail::operand_bytes(a_kc, M, K, lda, 2) > (1LL << 31) ||
        gemm_detail::operand_bytes(b_kc, N, K, ldb, 2) > (1LL << 31))
      return fail(GPT_ESHAPE, "gemm: each operand must span at most 2 GiB");
    const long long stride = (long long)M * N;
    const EpiSplit part{ws, stride, N};
    if (sp.big)
      gemm_detail::launch_dma<256, 256, 2, 4, EpiSplit, SITE>(a_kc, b_kc, M, N, K, A, lda, B, ldb, part, s, sp.splits);
    else
      gemm_detail::launch_dma<128, 128, 2, 2, EpiSplit, SITE>(a_kc, b_kc, M, N, K, A, lda, B, ldb, part, s, sp.splits);
    const int kps = (int)cdiv(cdiv(K, sp.splits), 64) * 64;
    const int used = (int)cdiv(K, kps);
    const long long n = (long long)M * (N / 4);
    gemm_detail::splitk_reduce_kernel<0><<<(unsigned)cdiv(n, 256), 256, 0, s>>>(ws, stride, used, epi.out,
                                                                            epi.ldo, M, N, epi.beta);
    return check_launch("gemm split-K");
  }
}

// Two fp32-output bf16 products with row-contiguous operands (weight gradients dW = dY^T X over
// the tokens) in one launch of 256 x 256 tiles, unsplit: for pairs whose tiles together fill
// about one round of the CUs while each alone would leave CUs idle or need split-K partials
// (the d32 q/k/v and out weight gradients: 192 + 64 tiles).  Same argument rules as gemm();
// both outputs overwrite or both accumulate (beta).
template <int SITE>
inline gpt_status gemm_wgrad_pair(int M0, int N0, int K0, const bf16* A0, long long lda0,
                                  const bf16* B0, long long ldb0, const EpiStoreF32& e0, int M1,
                                  int N1, int K1, const bf16* A1, long long lda1, const bf16* B1,
                                  long long ldb1, const EpiStoreF32& e1, hipStream_t s) {
  if (e0.beta != e1.beta) return fail(GPT_EINVAL, "gemm_wgrad_pair: both outputs take the same beta");
  const int Ms[2] = {M0, M1}, Ns[2] = {N0, N1}, Ks[2] = {K0, K1};
  const bf16* As[2] = {A0, A1};
  const bf16* Bs[2] = {B0, B1};
  const long long ldas[2] = {lda0, lda1}, ldbs[2] = {ldb0, ldb1};
  const EpiStoreF32* es[2] = {&e0, &e1};
  int tiles[2];
  for (int i = 0; i < 2; ++i) {
    if (Ms[i] <= 0 || Ns[i] <= 0 || Ks[i] <= 0 || Ks[i] % 8 || Ms[i] % 8 || Ns[i] % 8)
      return fail(GPT_ESHAPE, "gemm_wgrad_pair: M, N, K must be positive multiples of 8");
    if (ldas[i] % 8 || ldbs[i] % 8 || es[i]->ldo % 4)
      return fail(GPT_ESHAPE, "gemm_wgrad_pair: bad leading dimensions");
    if (((uintptr_t)As[i] | (uintptr_t)Bs[i] | (uintptr_t)es[i]->out) % 16)
      return fail(GPT_EINVAL, "gemm_wgrad_pair: operands must be 16-byte aligned");
    if (gemm_detail::operand_bytes(false, Ms[i], Ks[i], ldas[i], 2) > (1LL << 31) ||
        gemm_detail::operand_bytes(false, Ns[i], Ks[i], ldbs[i], 2) > (1LL << 31))
      return fail(GPT_ESHAPE, "gemm: each operand must span at most 2 GiB");
    tiles[i] = (int)(cdiv(Ms[i], 256) * cdiv(Ns[i], 256));
  }
  if (tiles[0] % 8) return fail(GPT_ESHAPE, "gemm_wgrad_pair: the first product needs a multiple of 8 tiles");
  auto go = [&](auto proto) -> gpt_status {
    using E = decltype(proto);
    gemm_detail::GemmProb<E> p[2];
    for (int i = 0; i < 2; ++i)
      p[i] = gemm_detail::GemmProb<E>{As[i], Bs[i], ldas[i], ldbs[i], Ms[i], Ns[i], Ks[i],
                         (uint32_t)gemm_detail::operand_bytes(false, Ms[i], Ks[i], ldas[i], 2),
                         (uint32_t)gemm_detail::operand_bytes(false, Ns[i], Ks[i], ldbs[i], 2),
                         E{es[i]->out, es[i]->ldo}, tiles[i]};
    gemm_detail::gemm_dma_pair_kernel<256, 256, 2, 4, 32, 4, false, false, E, SITE>
        <<<dim3((unsigned)(tiles[0] + tiles[1])), 64 * 2 * 4, 0, s>>>(p[0], p[1]);
    return check_launch("gemm_wgrad_pair");
  };
  return e0.beta ? go(EpiAccF32{}) : go(EpiPutF32{});
}

}  // namespace gpt
