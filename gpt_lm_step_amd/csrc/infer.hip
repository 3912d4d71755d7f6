// Inference with a key/value cache: GPT.forward with kv_cache and GPT.generate of the "$1000 tier
// nanochat run" discussion (nanochat #8).  Keys are cached after rotary and QK-norm, values as
// projected; a chunk of T new tokens per sequence at cache positions p0 .. p0+T-1 attends to
// every cached position before it and causally within itself (which covers the page's three
// cases: a full causal pass, a single query over the cache, and a chunk after a prefix).  The
// logits of each sequence's last position are softcapped; sampling keeps the logits at or above
// the k-th largest (top_k), divides by the temperature and draws by inverting the cumulative
// softmax in vocabulary order with a caller-supplied uniform number (temperature 0: argmax).
#include <math.h>

#include <algorithm>

#include "gemm.h"

struct gpt_infer {
  gpt_config cfg;
  int max_batch, max_seq, batch, pos;
  gpt::Layout L;
  void *cos_t, *sin_t, *kc, *vc;  // rotary tables [max_seq][hd/2]; caches [L][B][H][max_seq][hd]
  float *x, *rstd, *lse2, *xl;
  void *a, *qkv, *att, *act, *fl;
  float* part;     // split-attention partials [max_batch H AS_MAX_T splits][hd + 2]
  float* sk_part;  // skinny-GEMM split partials [splits][M][d_model], M <= SK_MAX_M
  int32_t* tok_c;
  int* err;
  gpt::Prof prof;  // per-launch timing (gpt_infer_profile)
};

namespace gpt {
namespace {

// Rotary embedding and QK-norm of the chunk's q and k (in place in qkv, as in training), with the
// token's rotated, normalised k and its v appended to the cache at position p0 + t.  One thread
// per 8 consecutive rotation pairs (i..i+7, i+half..i+half+7) of one q or k head, the hd/16
// lanes of a head reducing its sum of squares; the same thread copies one 8-element group of v.
// The rotary tables are those of positions p0.. (the caller offsets them).
template <typename T>
__global__ __launch_bounds__(256) void rope_append_kernel(T* __restrict__ qkv,
                                                          const T* __restrict__ cos_t,
                                                          const T* __restrict__ sin_t,
                                                          T* __restrict__ kc, T* __restrict__ vc,
                                                          int B, int Tn, int H, int hd, int p0,
                                                          int max_seq, int qk_norm, float eps) {
  const int D = H * hd, half = hd / 2, per_tok = D / 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long long)B * Tn * per_tok) return;  // whole lane groups of a head exit together
  const long long tok = gid / per_tok;
  const int p = (int)(gid % per_tok) * 8;
  const int hq = p / half, i = p % half, hh = hq % H;
  const int b = (int)(tok / Tn), t = (int)(tok % Tn);
  T* row = qkv + tok * 3 * D;
  T* base = row + (hq < H ? 0 : D) + hh * hd;
  float x1[8], x2[8], c[8], sn[8], y1[8], y2[8];
  // every load first (v's too), so the kernel makes one round trip to memory
  const vec8_t<T> v8 = load8(row + 2 * D + p);
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
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    y1[e] *= r;
    y2[e] *= r;
  }
  store8_f32(base + i, y1);
  store8_f32(base + i + half, y2);
  const long long slot = (((long long)b * H + hh) * max_seq + p0 + t) * hd;
  if (hq >= H) {
    store8_f32(kc + slot + i, y1);
    store8_f32(kc + slot + i + half, y2);
  }
  // v group p of this token: head p / hd, dims p % hd .. +8
  const long long vslot = (((long long)b * H + p / hd) * max_seq + p0 + t) * hd + p % hd;
  store8(vc + vslot, v8);
}

// Attention of up to AS_MAX_T new queries over the cache, split over the keys: workgroup
// (b H + h, u, s) takes keys [s AS_KEYS, (s + 1) AS_KEYS) of query (b, t = t0 + u) (those at
// positions <= p0 + t) and writes the split's running max m, sum l = sum exp(score - m) and
// unnormalised output o = sum exp(score - m) v to part[(((b H + h) Tq + u) S + s)][HD + 2]
// (Tq = gridDim.y queries from t0 of the chunk's Tn); attn_combine_kernel merges the splits.
// HD / 8 lanes share a key row (8 elements each), so each load instruction of a wave covers
// WAVE * 8 / HD whole rows, contiguous in the cache; a wave issues the loads of all its key and
// value rows at once (keys past the visible range load the last visible row and get weight 0).
constexpr int AS_KEYS = 128, AS_THREADS = 256, AS_MAX_T = 16;
template <typename T, int HD>
__global__ __launch_bounds__(AS_THREADS) void attn_split_kernel(const T* __restrict__ qkv,
                                                                const T* __restrict__ kc,
                                                                const T* __restrict__ vc,
                                                                float* __restrict__ part, int Tn,
                                                                int t0, int H, int p0, int max_seq,
                                                                int S, float scale) {
  constexpr int LPK = HD / 8, KPI = WAVE / LPK, NW = AS_THREADS / WAVE, KW = AS_KEYS / NW;
  constexpr int NR = KW / KPI;  // rows per lane
  static_assert(KW % KPI == 0 && AS_KEYS <= AS_THREADS, "key split shape");
  __shared__ float qs[HD], sc[AS_KEYS], red[NW * HD], wm[NW], wl[NW];
  const int bh = blockIdx.x, b = bh / H, h = bh % H, u = blockIdx.y, t = t0 + u, sp = blockIdx.z;
  const int k0 = sp * AS_KEYS, k1 = min(p0 + t + 1, k0 + AS_KEYS);
  const int D = H * HD;
  const long long tok = (long long)b * Tn + t;
  float* out = part + (((long long)bh * gridDim.y + u) * S + sp) * (HD + 2);
  if (k0 >= k1) {  // no key of this split is visible to the query
    if (threadIdx.x < HD) out[threadIdx.x] = 0.f;
    if (threadIdx.x == 0) { out[HD] = -INFINITY; out[HD + 1] = 0.f; }
    return;
  }
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
  const int g = lane / LPK, e0 = (lane % LPK) * 8;
  const T* K = kc + ((long long)b * H + h) * max_seq * HD;
  const T* V = vc + ((long long)b * H + h) * max_seq * HD;
  vec8_t<T> kr[NR], vr[NR];
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const int jc = min(k0 + w * KW + n * KPI + g, k1 - 1);
    kr[n] = load8(K + (long long)jc * HD + e0);
  }
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const int jc = min(k0 + w * KW + n * KPI + g, k1 - 1);
    vr[n] = load8(V + (long long)jc * HD + e0);
  }
  if (threadIdx.x < HD) qs[threadIdx.x] = to_f32(qkv[tok * 3 * D + h * HD + threadIdx.x]) * scale;
  __syncthreads();
  float q8[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) q8[e] = qs[e0 + e];
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const int j = k0 + w * KW + n * KPI + g;
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += q8[e] * to_f32(kr[n][e]);
#pragma unroll
    for (int o = LPK / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, WAVE);
    if (lane % LPK == 0) sc[w * KW + n * KPI + g] = j < k1 ? dot : -INFINITY;
  }
  __syncthreads();
  const float sv = threadIdx.x < AS_KEYS ? sc[threadIdx.x] : -INFINITY;
  float m = wave_max(sv);
  if (lane == 0) wm[w] = m;
  __syncthreads();
  m = wm[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) m = fmaxf(m, wm[i]);
  const float ev = sv == -INFINITY ? 0.f : __expf(sv - m);
  if (threadIdx.x < AS_KEYS) sc[threadIdx.x] = ev;
  const float ls = wave_sum(ev);
  if (lane == 0) wl[w] = ls;
  __syncthreads();
  float o8[8] = {};
#pragma unroll
  for (int n = 0; n < NR; ++n) {
    const float pj = sc[w * KW + n * KPI + g];
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] += pj * to_f32(vr[n][e]);
  }
#pragma unroll
  for (int o = LPK; o < WAVE; o <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e) o8[e] += __shfl_xor(o8[e], o, WAVE);
  if (g == 0)
#pragma unroll
    for (int e = 0; e < 8; ++e) red[w * HD + e0 + e] = o8[e];
  __syncthreads();
  if (threadIdx.x < HD) {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) acc += red[i * HD + threadIdx.x];
    out[threadIdx.x] = acc;
  }
  if (threadIdx.x == 0) {
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) l += wl[i];
    out[HD] = m;
    out[HD + 1] = l;
  }
}

// out[b, t0 + u, h, :] = sum_s exp(m_s - M) o_s / sum_s exp(m_s - M) l_s, M = max_s m_s
// (splits in order); one workgroup per (b H + h, u), u < Tq, one thread per head dimension.
template <typename T>
__global__ void attn_combine_kernel(const float* __restrict__ part, T* __restrict__ out, int Tn,
                                    int t0, int Tq, int H, int hd, int S) {
  const int q = blockIdx.x, d = threadIdx.x;
  if (d >= hd) return;
  const float* p = part + (long long)q * S * (hd + 2);
  // (unrolled so that a group of splits' loads is in flight together)
  float M = -INFINITY;
#pragma unroll 8
  for (int s = 0; s < S; ++s) M = fmaxf(M, p[s * (hd + 2) + hd]);
  float L = 0.f, acc = 0.f;
#pragma unroll 8
  for (int s = 0; s < S; ++s) {
    const float ms = p[s * (hd + 2) + hd];
    const float wgt = ms == -INFINITY ? 0.f : __expf(ms - M);
    L += wgt * p[s * (hd + 2) + hd + 1];
    acc += wgt * p[s * (hd + 2) + d];
  }
  const int bh = q / Tq, t = t0 + q % Tq, b = bh / H, h = bh % H;
  out[((long long)b * Tn + t) * H * hd + h * hd + d] = from_f32<T>(acc / L);
}

// Skinny GEMM for decode steps: C[M, N] = A[M, K] W[N, K]^T with few rows of activations (bf16,
// K-contiguous), fp32 accumulation and the epilogues of gemm().  Every weight element is read
// once per call, so the kernel is bound by streaming W from HBM, and its speed by the weight
// bytes each CU keeps in flight.  Workgroup (x, y) owns the 32 output columns x*32.. and the K
// range [y Kr, (y+1) Kr), Kr = K / S.  Its SK_WAVES waves split that range; each issues the
// buffer loads of its weight rows for up to SK_CHUNK MFMA steps at once (registers hold weights
// only), while the workgroup stages the activations' slice [M][Kr] in LDS.  Products use
// v_mfma_f32_32x32x16_bf16 with the weight rows first, so that lane l ends with output row
// m = l % 32 and, in registers 4q..4q+3, columns q*8 + (l/32)*4 + 0..3 (rows m >= M are zero
// operands).  The waves' sums meet in LDS in a fixed order.  With S > 1 splits the epilogue is
// EpiSplit (split y writes its own fp32 partial) and the consumer adds the partials in order.
constexpr int SK_WAVES = 8, SK_CHUNK = 16, SK_MAX_SPLITS = 4, SK_MAX_M = 32;
constexpr int SK_LDS_A = 64 * 1024;  // bytes for the staged activations
template <class Epi>
__global__ __launch_bounds__(SK_WAVES * WAVE) void skinny_gemm_kernel(const bf16* __restrict__ A,
                                                                      long long lda, int M,
                                                                      const bf16* __restrict__ W,
                                                                      long long ldw, int K,
                                                                      Epi epi) {
  extern __shared__ __align__(16) unsigned char sk_smem[];
  bf16* As = reinterpret_cast<bf16*>(sk_smem);
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
  const int r = lane % 32, h = lane / 32;
  const int n0 = blockIdx.x * 32;
  const int Kr = K / gridDim.y, kr0 = blockIdx.y * Kr, kw = Kr / SK_WAVES, kb = w * kw;
  const int pitch = Kr + 8;  // LDS row pitch (elements)
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(W + (long long)n0 * ldw, (uint32_t)(32 * ldw * 2));
  const uint32_t ow = (uint32_t)((r * ldw + kr0 + kb + h * 8) * 2);
  constexpr int NB = SK_CHUNK;
  bf16x8 wf[NB];
  const int steps = kw / 16;
  auto issue = [&](int s0) {
#pragma unroll
    for (int u = 0; u < NB; ++u)
      if (s0 + u < steps) wf[u] = bload8<bf16>(rw, ow + (uint32_t)((s0 + u) * 16) * 2);
  };
  issue(0);
  // activations [M][Kr] -> LDS (16-byte pieces), while the weight loads are in flight
  {
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)(M * lda * 2));
    const int per_row = Kr / 8;
    for (int i = threadIdx.x; i < M * per_row; i += SK_WAVES * WAVE) {
      const int m = i / per_row, c8 = (i % per_row) * 8;
      *reinterpret_cast<bf16x8*>(As + m * pitch + c8) =
          bload8<bf16>(ra, (uint32_t)((m * lda + kr0 + c8) * 2));
    }
  }
  __syncthreads();
  f32x16 acc = {};
  for (int s0 = 0; s0 < steps; s0 += NB) {
    if (s0 > 0) issue(s0);
#pragma unroll
    for (int u = 0; u < NB; ++u) asm volatile("" : "+v"(wf[u]));
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (s0 + u < steps) {
        bf16x8 af = {};
        if (r < M) af = *reinterpret_cast<const bf16x8*>(As + r * pitch + kb + (s0 + u) * 16 + h * 8);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[u], af, acc, 0, 0, 0);
      }
    }
  }
  __syncthreads();  // the staging area becomes the reduction buffer
  float* red = reinterpret_cast<float*>(sk_smem);
#pragma unroll
  for (int i = 0; i < 16; ++i) red[(w * 16 + i) * WAVE + lane] = acc[i];
  __syncthreads();
  if (w != 0 || r >= M) return;
  float sum[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    sum[i] = red[i * WAVE + lane];
#pragma unroll
    for (int v = 1; v < SK_WAVES; ++v) sum[i] += red[(v * 16 + i) * WAVE + lane];
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float v4[4] = {sum[4 * q], sum[4 * q + 1], sum[4 * q + 2], sum[4 * q + 3]};
    epi(r, n0 + q * 8 + h * 4, v4);
  }
}

// LDS bytes of a skinny launch: the staged activations, at least the reduction buffer.
inline size_t skinny_lds(int M, int K, int S) {
  return std::max((size_t)M * (K / S + 8) * 2, (size_t)SK_WAVES * 16 * WAVE * 4);
}

// Whether a bf16 product of these sizes runs on the skinny kernel with S splits of K.
inline bool skinny_ok(int M, int N, int K, long long lda, long long ldw, int S = 1) {
  return M >= 1 && M <= SK_MAX_M && N % 32 == 0 && K % (S * 16 * SK_WAVES) == 0 && lda % 8 == 0 &&
         ldw % 8 == 0 && (long long)M * lda * 2 < (1LL << 31) && 32LL * ldw * 2 < (1LL << 31) &&
         (size_t)M * (K / S + 8) * 2 <= (size_t)SK_LDS_A;
}

// Splits of K for a product with lda = ldw = K: the fewest (a power of two, at most
// SK_MAX_SPLITS) that give at least 512 workgroups and fit the activations' slice in LDS, while
// every wave keeps a multiple of 16 of K (0 when the skinny kernel cannot take the product).
inline int skinny_splits(int M, int N, int K) {
  for (int S = 1; S <= SK_MAX_SPLITS; S *= 2) {
    if (K % (S * 16 * SK_WAVES)) return 0;
    const bool fits = skinny_ok(M, N, K, K, K, S);
    if (fits && ((long long)(N / 32) * S >= 512 || S == SK_MAX_SPLITS || K % (2 * S * 16 * SK_WAVES)))
      return S;
  }
  return 0;
}

// Decode-sized products go to the skinny kernel (one split, the epilogue applied in place);
// everything else (prefill, fp32) to gemm().
template <int SITE, typename T, class Epi>
gpt_status infer_gemm(int M, int N, int K, const T* A, long long lda, const T* W, long long ldw,
                      const Epi& epi, hipStream_t s) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (skinny_ok(M, N, K, lda, ldw)) {
      const size_t lds = skinny_lds(M, K, 1);
      if constexpr (std::is_same<Epi, EpiStoreF32>::value)
        skinny_gemm_kernel<<<N / 32, SK_WAVES * WAVE, lds, s>>>(A, lda, M, W, ldw, K,
                                                               EpiPutF32{epi.out, epi.ldo});
      else
        skinny_gemm_kernel<<<N / 32, SK_WAVES * WAVE, lds, s>>>(A, lda, M, W, ldw, K, epi);
      return check_launch("skinny gemm");
    }
  }
  return gemm<SITE, T>(true, true, M, N, K, A, lda, W, ldw, epi, s);
}

// Residual update from split partials, then RMSNorm, one workgroup per row (M <= SK_MAX_M rows,
// D <= 256 * 8 * RR_MAXIT): x += sum_s part[s] (splits in order), rstd = 1/sqrt(mean(x^2) + eps),
// y = x * rstd in T.  Thread x owns columns x*8.. (+ 2048 per further pass); every split's loads
// of a pass are issued together.
constexpr int RR_MAXIT = 4;
template <typename T>
__global__ __launch_bounds__(256) void resid_rms_kernel(float* __restrict__ x,
                                                        const float* __restrict__ part, int S,
                                                        T* __restrict__ y,
                                                        float* __restrict__ rstd, int M, int D,
                                                        float eps) {
  __shared__ float red[256 / WAVE];
  const int row = blockIdx.x;
  const long long pstride = (long long)M * D;
  float* xr = x + (long long)row * D;
  float xs[RR_MAXIT][8];
  float ss = 0.f;
#pragma unroll
  for (int it = 0; it < RR_MAXIT; ++it) {
    const int cidx = (it * 256 + threadIdx.x) * 8;
    if (cidx < D) {
      float acc[8];
      load8_f32(xr + cidx, xs[it]);
      load8_f32(part + (long long)row * D + cidx, acc);
#pragma unroll
      for (int sp = 1; sp < SK_MAX_SPLITS; ++sp) {
        if (sp < S) {
          float p8[8];
          load8_f32(part + sp * pstride + (long long)row * D + cidx, p8);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[e] += p8[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xs[it][e] += acc[e];
        ss += xs[it][e] * xs[it][e];
      }
      store8_f32(xr + cidx, xs[it]);
    }
  }
  ss = wave_sum(ss);
  if (threadIdx.x % WAVE == 0) red[threadIdx.x / WAVE] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < 256 / WAVE; ++i) tot += red[i];
  const float r = 1.f / sqrtf(tot / (float)D + eps);
  if (threadIdx.x == 0) rstd[row] = r;
#pragma unroll
  for (int it = 0; it < RR_MAXIT; ++it) {
    const int cidx = (it * 256 + threadIdx.x) * 8;
    if (cidx < D) {
#pragma unroll
      for (int e = 0; e < 8; ++e) xs[it][e] *= r;
      store8_f32(y + (long long)row * D + cidx, xs[it]);
    }
  }
}

// x += A W^T followed by y = RMSNorm(x) for a decode-sized product, in two launches: the skinny
// kernel's split partials (skinny_split, which returns the split count), then resid_rms_kernel.
template <typename T>
gpt_status skinny_split(gpt_infer* c, int M, int N, int K, const T* A, const T* W, int* S_out,
                        hipStream_t s) {
  if constexpr (!std::is_same<T, bf16>::value) {
    return fail(GPT_EINVAL, "skinny gemm: bf16 only");
  } else {
    const int S = skinny_splits(M, N, K);
    if (S < 1 || !skinny_ok(M, N, K, K, K, S) ||
        (long long)S * M * N > (long long)SK_MAX_SPLITS * SK_MAX_M * c->cfg.d_model)
      return fail(GPT_EINVAL, "skinny gemm: no split of K fits");
    skinny_gemm_kernel<<<dim3(N / 32, S), SK_WAVES * WAVE, skinny_lds(M, K, S), s>>>(
        A, K, M, W, K, K, EpiSplit{c->sk_part, (long long)M * N, (long long)N});
    *S_out = S;
    return check_launch("skinny gemm (split)");
  }
}
template <typename T>
gpt_status resid_rms(gpt_infer* c, int M, int N, int S, T* y, hipStream_t s) {
  resid_rms_kernel<T><<<M, 256, 0, s>>>(c->x, c->sk_part, S, y, c->rstd, M, N, c->cfg.rms_eps);
  return check_launch("residual + rmsnorm");
}

// xl[b] = x[b * Tn + Tn - 1]: the residual stream at each sequence's last position.
__global__ void gather_last_kernel(const float* __restrict__ x, float* __restrict__ xl, int B,
                                   int Tn, int D) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)B * D) return;
  const long long b = i / D, d = i % D;
  xl[i] = x[(b * Tn + Tn - 1) * D + d];
}

// logits = cap * tanh(logits / cap) in place (cap 0: unchanged).
__global__ void softcap_kernel(float* __restrict__ z, long long n, float cap) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n && cap > 0.f) z[i] = cap * tanhf(z[i] / cap);
}

// Order-preserving unsigned key of a float (larger float, larger key) and its inverse.  Only the
// negative NaN with every mantissa bit set maps to 0, which marks the columns past the row's end.
__device__ __forceinline__ uint32_t fkey(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

constexpr int SAMPLE_THREADS = 1024;

__device__ __forceinline__ float block_sum_1k(float v, float* sm) {
  v = wave_sum(v);
  __syncthreads();
  if (threadIdx.x % WAVE == 0) sm[threadIdx.x / WAVE] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < SAMPLE_THREADS / WAVE; ++i) t += sm[i];
  return t;
}

// One workgroup per row; thread x holds the keys of columns [x * PER, (x + 1) * PER) (vocabulary
// order), 0 past the row's end, so that every per-column test is one unsigned compare.
template <int PER>
__global__ __launch_bounds__(SAMPLE_THREADS) void sample_kernel(const float* __restrict__ logits,
                                                                int V, float temperature, int top_k,
                                                                const float* __restrict__ u,
                                                                int32_t* __restrict__ tokens) {
  __shared__ float sm[SAMPLE_THREADS / WAVE];
  __shared__ uint32_t km[SAMPLE_THREADS / WAVE];
  __shared__ int im[SAMPLE_THREADS / WAVE];
  const float* z = logits + (long long)blockIdx.x * V;
  const int c0 = threadIdx.x * PER;
  // buffer loads: one offset register with immediate steps; columns past the row read 0.0
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(z, (uint32_t)V * 4u);
  uint32_t key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i)
    key[i] = fkey(__uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)(c0 + i) * 4u, 0, 0)));
  if (c0 + PER > V) {
#pragma unroll
    for (int i = 0; i < PER; ++i) key[i] = c0 + i < V ? key[i] : 0u;
  }
  // phase boundary: the keys count as rewritten, so no per-column compare result (a 64-bit
  // mask each) is carried from one phase into the next
  auto fence_keys = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) asm volatile("" : "+v"(key[i]));
  };
  const int lane = threadIdx.x % WAVE, wv = threadIdx.x / WAVE;
  if (!(temperature > 0.f)) {
    // argmax, first index among equal maxima
    uint32_t bk = 0;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (key[i] > bk) { bk = key[i]; bi = c0 + i; }
    for (int o = 32; o >= 1; o >>= 1) {
      const uint32_t ok = __shfl_xor(bk, o, WAVE);
      const int oi = __shfl_xor(bi, o, WAVE);
      if (ok > bk || (ok == bk && oi < bi)) { bk = ok; bi = oi; }
    }
    if (lane == 0) { km[wv] = bk; im[wv] = bi; }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t k = km[0];
      int best = im[0];
      for (int i = 1; i < SAMPLE_THREADS / WAVE; ++i)
        if (km[i] > k || (km[i] == k && im[i] < best)) { k = km[i]; best = im[i]; }
      tokens[blockIdx.x] = min(best, V - 1);
    }
    return;
  }
  // top-k: the largest key tau with at least k columns >= tau (bit by bit from the top); keys at
  // or below that of -inf (the row's padding, -inf logits) are never kept
  uint32_t tau = 0;
  if (top_k > 0 && top_k < V) {
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = tau | (1u << bit);
      float cnt = 0.f;
#pragma unroll
      for (int i = 0; i < PER; ++i) cnt += key[i] >= cand ? 1.f : 0.f;
      if (block_sum_1k(cnt, sm) >= (float)top_k) tau = cand;
    }
  }
  tau = max(tau, fkey(-INFINITY) + 1u);
  fence_keys();
  // softmax of the kept logits / temperature
  const float inv_t = 1.f / temperature;
  uint32_t kmax = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) kmax = max(kmax, key[i]);
  for (int o = 32; o >= 1; o >>= 1) kmax = max(kmax, (uint32_t)__shfl_xor(kmax, o, WAVE));
  __syncthreads();
  if (lane == 0) km[wv] = kmax;
  __syncthreads();
  for (int i = 0; i < SAMPLE_THREADS / WAVE; ++i) kmax = max(kmax, km[i]);
  const float M = fkey_inv(kmax) * inv_t;
  fence_keys();
  // exp of a kept column, 0 for the others (recomputed where needed to keep registers low)
  // (branch-free: the exp is taken for every column and the compare only selects; a padding
  // key's NaN and a dropped column's value are discarded by the select)
  auto ex = [&](int i) {
    float e = __expf(fkey_inv(key[i]) * inv_t - M);
    asm volatile("" : "+v"(e));  // keeps the compiler from turning the select into a branch
    return key[i] >= tau ? e : 0.f;
  };
  float mine = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) mine += ex(i);
  // Cumulative sums in thread order (= vocabulary order).  Thread x owns the cell
  // [before + inc of the previous lane, before + its own inc): the edges are the same fp32 values
  // on both sides, so the cells tile [0, total) without gaps or overlaps.
  float inc = mine;
  for (int o = 1; o < WAVE; o <<= 1) {
    const float y = __shfl_up(inc, o, WAVE);
    if (lane >= o) inc += y;
  }
  const float prev = __shfl_up(inc, 1, WAVE);
  __syncthreads();
  if (lane == WAVE - 1) sm[wv] = inc;
  __syncthreads();
  float before = 0.f, total = 0.f;
  for (int i = 0; i < SAMPLE_THREADS / WAVE; ++i) {
    if (i == wv) before = total;
    total += sm[i];
  }
  const float start = lane == 0 ? before : before + prev, end = before + inc;
  const float target = u[blockIdx.x] * total;
  // the first column of the owning thread whose running sum exceeds the target, that thread's
  // last kept column when rounding of the running sum leaves none; the last kept column of the
  // row when the target rounds up to the total
  int pick = -1;
  fence_keys();  // recompute, do not keep, the exps
  if (target >= start && target < end) {
    // the running sums never decrease, so the first one above the target follows the count of
    // those at or below it (that column's exp is > 0)
    float run = start;
    int below = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      run += ex(i);
      below += run <= target ? 1 : 0;
    }
    if (below < PER) pick = c0 + below;
    else {  // rounding of the running sum: this thread's last kept column
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (ex(i) > 0.f) pick = c0 + i;
    }
  }
  for (int o = 32; o >= 1; o >>= 1) pick = max(pick, __shfl_xor(pick, o, WAVE));
  __syncthreads();
  if (lane == 0) im[wv] = pick;
  __syncthreads();
  int p = -1;
  for (int i = 0; i < SAMPLE_THREADS / WAVE; ++i) p = max(p, im[i]);
  if (p < 0) {  // the target rounded up to the total (uniform over the block): last kept column
    int last = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (key[i] >= tau) last = c0 + i;
    for (int o = 32; o >= 1; o >>= 1) last = max(last, __shfl_xor(last, o, WAVE));
    __syncthreads();
    if (lane == 0) im[wv] = last;
    __syncthreads();
    for (int i = 0; i < SAMPLE_THREADS / WAVE; ++i) p = max(p, im[i]);
  }
  if (threadIdx.x == 0) tokens[blockIdx.x] = p;
}

// Carves the context's buffers (or only measures them when base is null).
template <typename T>
void carve_infer(Carver& cv, gpt_infer* c) {
  const gpt_config& g = c->cfg;
  const long long D = g.d_model, F = g.d_mlp, H = g.n_head, hd = g.head_dim;
  const long long M = (long long)c->max_batch * c->max_seq;
  const long long cache = (long long)g.n_layer * c->max_batch * H * c->max_seq * hd;
  c->cos_t = cv.take<T>((size_t)c->max_seq * hd / 2);
  c->sin_t = cv.take<T>((size_t)c->max_seq * hd / 2);
  c->kc = cv.take<T>(cache);
  c->vc = cv.take<T>(cache);
  c->x = cv.take<float>(M * D);
  c->rstd = cv.take<float>(M);
  c->lse2 = cv.take<float>(M * H);
  c->xl = cv.take<float>((size_t)c->max_batch * D);
  c->a = cv.take<T>(M * D);
  c->qkv = cv.take<T>(M * 3 * D);
  c->att = cv.take<T>(M * D);
  c->act = cv.take<T>(M * F);
  c->fl = cv.take<T>((size_t)c->max_batch * D);
  c->sk_part = cv.take<float>((size_t)SK_MAX_SPLITS * SK_MAX_M * D);
  c->part = cv.take<float>((size_t)c->max_batch * H * AS_MAX_T * cdiv(c->max_seq, AS_KEYS) * (hd + 2));
  c->tok_c = cv.take<int32_t>(M);
  c->err = cv.take<int>(4);
}

template <typename T>
gpt_status infer_forward(gpt_infer* c, const T* P, const int32_t* tokens, int B, int Tn,
                         float* logits, hipStream_t s) {
  const gpt_config& g = c->cfg;
  const Layout& L = c->L;
  const int D = g.d_model, F = g.d_mlp, H = g.n_head, hd = g.head_dim, V = g.vocab;
  const long long M = (long long)B * Tn;
  const int p0 = c->pos;
  T *a = (T*)c->a, *qkv = (T*)c->qkv, *att = (T*)c->att, *act = (T*)c->act, *fl = (T*)c->fl;
  const T* cos_t = (const T*)c->cos_t + (long long)p0 * hd / 2;
  const T* sin_t = (const T*)c->sin_t + (long long)p0 * hd / 2;
  const long long layer_cache = (long long)c->max_batch * H * c->max_seq * hd;
  const double es = sizeof(T), Md = (double)M;
  Prof& prof = c->prof;
  // one launch (or a loop of one kind of launch); with profiling on, bracketed by events and
  // tagged with its algorithmic work: flops of its products, bytes it must move once
  auto run = [&](const char* name, double flops, double bytes, auto&& fn) -> gpt_status {
    if (!prof.on) return fn();
    hipEvent_t e0 = prof.get(), e1 = prof.get();
    if (!e0 || !e1) return fail(GPT_EHIP, "profiling: hipEventCreate failed");
    (void)hipEventRecord(e0, s);
    gpt_status st = fn();
    (void)hipEventRecord(e1, s);
    prof.recs.push_back({name, flops, bytes, e0, e1});
    return st;
  };
  auto mm = [](double m, double n, double k) { return 2.0 * m * n * k; };
#define TRY(x)                                 \
  do {                                         \
    gpt_status st_ = (x);                      \
    if (st_ != GPT_OK) return st_;             \
  } while (0)
  TRY(run("embed", 0, Md * D * (es + 4), [&] {
    return launch_embed_fwd<T>(tokens, P + L.wte, nullptr, c->x, c->rstd, c->tok_c, c->err, M, D, V,
                               g.rms_eps, s);
  }));
  // decode-sized steps: each residual product leaves the next product's normalised input
  const bool dec = std::is_same<T, bf16>::value && skinny_splits((int)M, D, D) > 0 &&
                   skinny_splits((int)M, D, F) > 0 && D <= 256 * 8 * RR_MAXIT;
  for (int l = 0; l < g.n_layer; ++l) {
    T* kc = (T*)c->kc + l * layer_cache;
    T* vc = (T*)c->vc + l * layer_cache;
    if (l == 0 || !dec)
      TRY(run("rmsnorm", 0, Md * D * (4 + es),
              [&] { return launch_rms_fwd<T>(c->x, a, c->rstd, M, D, g.rms_eps, s); }));
    TRY(run("qkv", mm(Md, 3.0 * D, D), (3.0 * D * D + Md * D + Md * 3 * D) * es, [&] {
      return infer_gemm<G_INF_QKV, T>((int)M, 3 * D, D, a, D, P + L.wqkv[l], D,
                                      EpiStore<T>{qkv, 3LL * D}, s);
    }));
    TRY(run("rope_append", 0, Md * 7 * D * es, [&] {
      rope_append_kernel<T><<<cdiv(M * D / 8, 256), 256, 0, s>>>(qkv, cos_t, sin_t, kc, vc, B, Tn,
                                                                  H, hd, p0, c->max_seq,
                                                                  g.qk_norm, g.rms_eps);
      return check_launch("rotary + cache append");
    }));
    if (p0 == 0 && Tn > AS_MAX_T) {
      // a first chunk: the training kernel's causal pass over the chunk itself
      const double pairs = (double)B * H * Tn * (Tn + 1) / 2.0;
      TRY(run("attention", 4.0 * pairs * hd, Md * 4 * D * es,
              [&] { return launch_attn_fwd<T>(qkv, att, c->lse2, B, Tn, H, hd, s, g.qk_norm); }));
    } else {
      // queries over the cache, AS_MAX_T at a time
      const float scale = 1.f / sqrtf((float)hd);
      for (int t0 = 0; t0 < Tn; t0 += AS_MAX_T) {
        const int tq = std::min(AS_MAX_T, Tn - t0), S = cdiv(p0 + t0 + tq, AS_KEYS);
        const double bh = (double)B * H, part_b = bh * tq * S * (hd + 2) * 4.0;
        double keys = 0;  // (query, visible key) pairs of the chunk
        for (int t = t0; t < t0 + tq; ++t) keys += p0 + t + 1;
        TRY(run("attn_split", 4.0 * bh * keys * hd,
                bh * (p0 + t0 + tq) * hd * 2 * es + bh * tq * hd * es + part_b, [&] {
                  const dim3 grid(B * H, tq, S);
                  if (hd == 128) attn_split_kernel<T, 128><<<grid, AS_THREADS, 0, s>>>(qkv, kc, vc, c->part, Tn, t0, H, p0, c->max_seq, S, scale);
                  else if (hd == 64) attn_split_kernel<T, 64><<<grid, AS_THREADS, 0, s>>>(qkv, kc, vc, c->part, Tn, t0, H, p0, c->max_seq, S, scale);
                  else attn_split_kernel<T, 32><<<grid, AS_THREADS, 0, s>>>(qkv, kc, vc, c->part, Tn, t0, H, p0, c->max_seq, S, scale);
                  return check_launch("attention (key splits)");
                }));
        TRY(run("attn_combine", 0, part_b + bh * tq * hd * es, [&] {
          attn_combine_kernel<T><<<B * H * tq, 128, 0, s>>>(c->part, att, Tn, t0, tq, H, hd, S);
          return check_launch("attention (combine)");
        }));
      }
    }
    int S = 0;
    if (dec) {
      const double sp = (double)skinny_splits((int)M, D, D);
      TRY(run("out", mm(Md, D, D), (1.0 * D * D + Md * D) * es + sp * Md * D * 4,
              [&] { return skinny_split<T>(c, (int)M, D, D, att, P + L.wo[l], &S, s); }));
      TRY(run("out_resid_norm", 0, (S + 2.0) * Md * D * 4 + Md * D * es,
              [&] { return resid_rms<T>(c, (int)M, D, S, a, s); }));
    } else {
      TRY(run("out", mm(Md, D, D), (1.0 * D * D + Md * D) * es + 2 * Md * D * 4, [&] {
        return infer_gemm<G_INF_OUT, T>((int)M, D, D, att, D, P + L.wo[l], D,
                                        EpiResid{c->x, c->x, (long long)D}, s);
      }));
      TRY(run("rmsnorm", 0, Md * D * (4 + es),
              [&] { return launch_rms_fwd<T>(c->x, a, c->rstd, M, D, g.rms_eps, s); }));
    }
    TRY(run("up", mm(Md, F, D), (1.0 * F * D + Md * D + Md * F) * es, [&] {
      return infer_gemm<G_INF_UP, T>((int)M, F, D, a, D, P + L.wfc[l], D,
                                     EpiRelu2<T>{act, (long long)F}, s);
    }));
    if (dec) {
      const double sp = (double)skinny_splits((int)M, D, F);
      TRY(run("down", mm(Md, D, F), (1.0 * D * F + Md * F) * es + sp * Md * D * 4,
              [&] { return skinny_split<T>(c, (int)M, D, F, act, P + L.wpr[l], &S, s); }));
      TRY(run("down_resid_norm", 0, (S + 2.0) * Md * D * 4 + Md * D * es,
              [&] { return resid_rms<T>(c, (int)M, D, S, a, s); }));
    } else {
      TRY(run("down", mm(Md, D, F), (1.0 * D * F + Md * F) * es + 2 * Md * D * 4, [&] {
        return infer_gemm<G_INF_DOWN, T>((int)M, D, F, act, F, P + L.wpr[l], F,
                                         EpiResid{c->x, c->x, (long long)D}, s);
      }));
    }
  }
  const double Bd = B;
  TRY(run("gather_last", 0, Bd * D * 8, [&] {
    gather_last_kernel<<<cdiv((long long)B * D, 256), 256, 0, s>>>(c->x, c->xl, B, Tn, D);
    return check_launch("gather last positions");
  }));
  TRY(run("final_norm", 0, Bd * D * (4 + es),
          [&] { return launch_rms_fwd<T>(c->xl, fl, c->rstd, B, D, g.rms_eps, s); }));
  TRY(run("head", mm(Bd, V, D), (1.0 * V * D + Bd * D) * es + Bd * V * 4, [&] {
    return infer_gemm<G_INF_HEAD, T>(B, V, D, fl, D, P + L.lm_head, D,
                                     EpiStoreF32{logits, (long long)V, 0}, s);
  }));
  TRY(run("softcap", 0, Bd * V * 8, [&] {
    softcap_kernel<<<cdiv((long long)B * V, 256), 256, 0, s>>>(logits, (long long)B * V, g.softcap);
    return check_launch("softcap");
  }));
#undef TRY
  return check_launch("inference forward");
}

}  // namespace
}  // namespace gpt

using namespace gpt;

extern "C" {

gpt_status gpt_infer_workspace_bytes(const gpt_config* cfg, int32_t max_batch, int32_t max_seq,
                                     size_t* bytes) {
  gpt_status st = validate(cfg);
  if (st != GPT_OK) return st;
  if (!bytes) return fail(GPT_EINVAL, "gpt_infer_workspace_bytes: bytes is null");
  if (max_batch < 1 || max_seq < 1 || max_seq > 8192)
    return fail(GPT_ESHAPE, "inference: 1 <= max_batch and 1 <= max_seq <= 8192");
  gpt_infer c{};
  c.cfg = *cfg;
  c.max_batch = max_batch;
  c.max_seq = max_seq;
  Carver cv(nullptr, 0);
  if (cfg->dtype == GPT_BF16) carve_infer<bf16>(cv, &c);
  else carve_infer<float>(cv, &c);
  *bytes = cv.size();
  return GPT_OK;
}

gpt_status gpt_infer_init(const gpt_config* cfg, int32_t max_batch, int32_t max_seq,
                          void* workspace, size_t ws_bytes, hipStream_t stream, gpt_infer** out) {
  size_t need = 0;
  gpt_status st = gpt_infer_workspace_bytes(cfg, max_batch, max_seq, &need);
  if (st != GPT_OK) return st;
  if (!out) return fail(GPT_EINVAL, "gpt_infer_init: out is null");
  if (cfg->has_x0_add || cfg->has_v_add || cfg->has_trigram)
    return fail(GPT_EINVAL, "inference: the table addends are not supported");
  if (!workspace || (uintptr_t)workspace % 256 || ws_bytes < need)
    return fail(GPT_EWORKSPACE, "gpt_infer_init: workspace missing, misaligned or too small");
  gpt_infer* c = new gpt_infer{};
  c->cfg = *cfg;
  c->max_batch = max_batch;
  c->max_seq = max_seq;
  c->batch = 0;
  c->pos = 0;
  c->L = make_layout(*cfg);
  Carver cv(workspace, ws_bytes);
  if (cfg->dtype == GPT_BF16) {
    carve_infer<bf16>(cv, c);
    st = launch_rope_table<bf16>((bf16*)c->cos_t, (bf16*)c->sin_t, max_seq, cfg->head_dim,
                                 cfg->rope_base, stream);
  } else {
    carve_infer<float>(cv, c);
    st = launch_rope_table<float>((float*)c->cos_t, (float*)c->sin_t, max_seq, cfg->head_dim,
                                  cfg->rope_base, stream);
  }
  if (st == GPT_OK) st = launch_fill((float*)c->err, 1, 0.f, stream);  // no problems seen yet
  if (st != GPT_OK) {
    delete c;
    return st;
  }
  *out = c;
  return GPT_OK;
}

gpt_status gpt_infer_reset(gpt_infer* ctx) {
  if (!ctx) return fail(GPT_EINVAL, "gpt_infer_reset: null context");
  ctx->pos = 0;
  ctx->batch = 0;
  return GPT_OK;
}

int32_t gpt_infer_position(const gpt_infer* ctx) { return ctx ? ctx->pos : -1; }

gpt_status gpt_infer_forward(gpt_infer* ctx, const void* params, const int32_t* tokens,
                             int32_t B, int32_t T, float* logits, hipStream_t stream) {
  if (!ctx || !params || !tokens || !logits) return fail(GPT_EINVAL, "gpt_infer_forward: null argument");
  if (B < 1 || B > ctx->max_batch || T < 1) return fail(GPT_ESHAPE, "gpt_infer_forward: 1 <= B <= max_batch, T >= 1");
  if (ctx->pos > 0 && B != ctx->batch)
    return fail(GPT_ESHAPE, "gpt_infer_forward: the batch size is fixed until gpt_infer_reset");
  if ((long long)ctx->pos + T > ctx->max_seq) return fail(GPT_ERANGE, "gpt_infer_forward: the cache is full");
  if (((uintptr_t)params | (uintptr_t)logits) % 16) return fail(GPT_EINVAL, "gpt_infer_forward: misaligned buffer");
  gpt_status st = ctx->cfg.dtype == GPT_BF16
                      ? infer_forward<bf16>(ctx, (const bf16*)params, tokens, B, T, logits, stream)
                      : infer_forward<float>(ctx, (const float*)params, tokens, B, T, logits, stream);
  if (st != GPT_OK) return st;
  ctx->batch = B;
  ctx->pos += T;
  return GPT_OK;
}

gpt_status gpt_sample(const float* logits, int32_t B, int32_t V, float temperature, int32_t top_k,
                      const float* uniforms, int32_t* tokens, hipStream_t stream) {
  if (B == 0) return GPT_OK;
  if (!logits || !tokens || (temperature > 0.f && !uniforms)) return fail(GPT_EINVAL, "gpt_sample: null argument");
  if (B < 0 || V < 1 || V > 65536) return fail(GPT_ESHAPE, "gpt_sample: 1 <= V <= 65536");
  if (!(temperature >= 0.f) || top_k < 0) return fail(GPT_ERANGE, "gpt_sample: temperature >= 0, top_k >= 0");
  if (V <= 16 * SAMPLE_THREADS)
    sample_kernel<16><<<B, SAMPLE_THREADS, 0, stream>>>(logits, V, temperature, top_k, uniforms, tokens);
  else
    sample_kernel<64><<<B, SAMPLE_THREADS, 0, stream>>>(logits, V, temperature, top_k, uniforms, tokens);
  return check_launch("sample");
}

gpt_status gpt_infer_check_errors(gpt_infer* ctx, hipStream_t stream, int32_t* flags) {
  if (!ctx || !flags) return fail(GPT_EINVAL, "gpt_infer_check_errors: null argument");
  int32_t h = 0;
  if (hipMemcpyAsync(&h, ctx->err, sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(GPT_EHIP, "gpt_infer_check_errors: copy failed");
  *flags = h;
  return launch_fill((float*)ctx->err, 1, 0.f, stream);
}

gpt_status gpt_infer_profile(gpt_infer* ctx, int32_t enable) {
  if (!ctx) return fail(GPT_EINVAL, "gpt_infer_profile: null context");
  ctx->prof.on = enable != 0;
  return GPT_OK;
}

gpt_status gpt_infer_profile_read(gpt_infer* ctx, gpt_profile_entry* out, int32_t* count) {
  if (!ctx || !count) return fail(GPT_EINVAL, "gpt_infer_profile_read: null argument");
  return prof_read(ctx->prof, out, count, "gpt_infer_profile_read");
}

gpt_status gpt_infer_destroy(gpt_infer* ctx) {
  delete ctx;
  return GPT_OK;
}

}  // extern "C"
