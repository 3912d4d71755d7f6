// Matrix-core GEMMs of the step (q/k/v, out, MLP up/down and LM-head projections and their
// input- and weight-gradients), hand-written for gfx950.
//
//   C[m, n] = sum_k A(m, k) * B(n, k)
//
// Each operand is either K-contiguous ("KC": element (r, k) at p[r*ld + k]) or row-contiguous
// ("RC": element (r, k) at p[k*ld + r]).  Forward projections y = x W^T are KC x KC; input
// gradients dx = dy W are KC x RC; weight gradients dW = dy^T x are RC x RC.
//
// Design (one 256-thread workgroup per 128x128 output tile, 4 waves of 64x64):
//  * tiles of A and B are staged through LDS as [row][k] with 16 bytes of padding per row;
//    global loads are 16 B vectors, coalesced along the contiguous dimension; RC operands are
//    transposed on the way in by an 8x8 in-register transpose, so both layouts feed the same
//    LDS format;
//  * the next K tile is loaded into registers while the current one is multiplied (two LDS
//    buffers, one barrier per K step);
//  * bf16 uses v_mfma_f32_32x32x16_bf16, fp32 uses v_mfma_f32_32x32x2f32 (8 per 16-wide K
//    slice); both take 8 consecutive K values per lane, so operand fragments are identical;
//  * the tile order keeps each XCD on a contiguous block of output tiles (L2 reuse), grouped
//    along M so neighbouring tiles share operand panels;
//  * epilogues are fused: bf16/fp32 stores, value addend, ReLU^2 (+ pre-activation),
//    dReLU^2, residual add, and beta-accumulation for weight gradients.
// Header-only: every call site instantiates its own kernel symbol (a GemmSite tag), so
// profiles name the projection a launch belongs to.
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

// Call sites of the GEMM: each gets its own kernel symbol, so profiles name the projection.
enum GemmSite {
  G_TEST = 0, G_QKV, G_OUT, G_UP, G_DOWN, G_HEAD, G_HEAD_DGRAD, G_HEAD_WGRAD, G_DOWN_DGRAD,
  G_DOWN_WGRAD, G_UP_DGRAD, G_UP_WGRAD, G_OUT_DGRAD, G_OUT_WGRAD, G_QKV_DGRAD, G_QKV_WGRAD,
  G_TRI, G_TRI_WGRAD
};

namespace gemm_detail {

constexpr int BM = 128, BN = 128, THREADS = 256;

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

// Global -> registers -> LDS staging of one ROWS x BK operand tile.
template <typename T, int ROWS, bool KC>
struct Stage {
  using C = Cfg<T>;
  using V = vec8_t<T>;
  static constexpr int NVEC = ROWS * C::KV;                       // KC: vectors per tile
  static constexpr int PER = KC ? (NVEC + THREADS - 1) / THREADS : 8;
  static constexpr int NBLK = (C::BK / 8) * (ROWS / 8);           // RC: 8x8 blocks per tile
  static_assert(KC || NBLK <= THREADS, "one 8x8 block per thread at most");
  V r[PER];

  __device__ __forceinline__ void load(const T* __restrict__ p, long long ld, int row0, int k0,
                                       int rows_lim, int k_lim) {
    const int tid = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int v = tid + i * THREADS;
        const int row = row0 + v / C::KV, k = k0 + (v % C::KV) * 8;
        if (v < NVEC && row < rows_lim && k < k_lim) r[i] = load8(p + (long long)row * ld + k);
        else r[i] = V{};
      }
    } else {
      if (tid < NBLK) {
        const int kb = tid / (ROWS / 8), rb = tid % (ROWS / 8);
        const int row = row0 + rb * 8;
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          const int k = k0 + kb * 8 + kk;
          if (row < rows_lim && k < k_lim) r[kk] = load8(p + (long long)k * ld + row);
          else r[kk] = V{};
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
        if (v < NVEC) store8(lds + (v / C::KV) * C::PITCH + (v % C::KV) * 8, r[i]);
      }
    } else {
      if (tid < NBLK) {
        const int kb = tid / (ROWS / 8), rb = tid % (ROWS / 8);
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) {
          V o;
#pragma unroll
          for (int kk = 0; kk < 8; ++kk) o[kk] = r[kk][rr];
          store8(lds + (rb * 8 + rr) * C::PITCH + kb * 8, o);
        }
      }
    }
  }
};

// Logical tile order: blocks are dispatched round-robin over the 8 XCDs, so block b runs on
// XCD b % 8.  Give XCD x the contiguous range of logical tiles x*per .. x*per+per-1, and walk
// tiles in groups of GROUP_M row-tiles so that consecutive tiles share A and B panels.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP_M = 8;
  const int nb = gridDim.x, b = blockIdx.x;
  const int L = (nb % 8 == 0) ? (b % 8) * (nb / 8) + b / 8 : b;
  const int per_group = GROUP_M * tiles_n;
  const int grp = L / per_group;
  const int first_m = grp * GROUP_M;
  const int gm = min(tiles_m - first_m, GROUP_M);
  const int in = L % per_group;
  tm = first_m + in % gm;
  tn = in / gm;
}

template <typename T, bool A_KC, bool B_KC, class Epi, int SITE>
__global__ __launch_bounds__(THREADS, 2) void gemm_kernel(const T* __restrict__ A, long long lda,
                                                          const T* __restrict__ B, long long ldb,
                                                          int M, int N, int K, Epi epi) {
  using C = Cfg<T>;
  __shared__ __attribute__((aligned(16))) T lds[2][(BM + BN) * C::PITCH];
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
  const int wm = (w / 2) * 64, wn = (w % 2) * 64;
  const int lr = lane % 32, lg = lane / 32;

  Stage<T, BM, A_KC> sa;
  Stage<T, BN, B_KC> sb;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  const int nk = (K + C::BK - 1) / C::BK;
  sa.load(A, lda, m0, 0, M, K);
  sb.load(B, ldb, n0, 0, N, K);
  sa.store(lds[0]);
  sb.store(lds[0] + BM * C::PITCH);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      sa.load(A, lda, m0, (kt + 1) * C::BK, M, K);
      sb.load(B, ldb, n0, (kt + 1) * C::BK, N, K);
    }
    const T* As = lds[cur];
    const T* Bs = lds[cur] + BM * C::PITCH;
#pragma unroll
    for (int ks = 0; ks < C::BK; ks += 16) {
      vec8_t<T> af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = load8(As + (wm + i * 32 + lr) * C::PITCH + ks + lg * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j) bfr[j] = load8(Bs + (wn + j * 32 + lr) * C::PITCH + ks + lg * 8);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) Mma<T>::run(acc[i][j], af[i], bfr[j]);
    }
    if (kt + 1 < nk) {
      sa.store(lds[cur ^ 1]);
      sb.store(lds[cur ^ 1] + BM * C::PITCH);
    }
    __syncthreads();
  }

  // C layout of a 32x32 MFMA tile: lane l, register r -> row (r/4)*8 + (l/32)*4 + r%4, col l%32.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int col = n0 + wn + j * 32 + lr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm + i * 32 + (r / 4) * 8 + lg * 4 + (r % 4);
        if (row < M) epi(row, col, acc[i][j][r]);
      }
    }
}

}  // namespace gemm_detail

template <int SITE, typename T, class Epi>
inline gpt_status gemm(bool a_kc, bool b_kc, int M, int N, int K, const T* A, long long lda, const T* B,
                long long ldb, const Epi& epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return GPT_OK;
  if (K <= 0 || K % 8) return fail(GPT_ESHAPE, "gemm: K must be a positive multiple of 8");
  if (lda % 8 || ldb % 8) return fail(GPT_ESHAPE, "gemm: leading dimensions must be multiples of 8");
  if ((!a_kc && M % 8) || (!b_kc && N % 8))
    return fail(GPT_ESHAPE, "gemm: row-contiguous operands need a multiple of 8 rows");
  if (((uintptr_t)A | (uintptr_t)B) % 16) return fail(GPT_EINVAL, "gemm: operands must be 16-byte aligned");
  const long long tiles = (long long)cdiv(M, gemm_detail::BM) * cdiv(N, gemm_detail::BN);
  if (tiles >= (1LL << 31)) return fail(GPT_ESHAPE, "gemm: too many tiles");
  dim3 grid((unsigned)tiles);
  if (a_kc && b_kc) gemm_detail::gemm_kernel<T, true, true, Epi, SITE><<<grid, gemm_detail::THREADS, 0, s>>>(A, lda, B, ldb, M, N, K, epi);
  else if (a_kc) gemm_detail::gemm_kernel<T, true, false, Epi, SITE><<<grid, gemm_detail::THREADS, 0, s>>>(A, lda, B, ldb, M, N, K, epi);
  else if (b_kc) gemm_detail::gemm_kernel<T, false, true, Epi, SITE><<<grid, gemm_detail::THREADS, 0, s>>>(A, lda, B, ldb, M, N, K, epi);
  else gemm_detail::gemm_kernel<T, false, false, Epi, SITE><<<grid, gemm_detail::THREADS, 0, s>>>(A, lda, B, ldb, M, N, K, epi);
  return check_launch("gemm");
}


}  // namespace gpt
