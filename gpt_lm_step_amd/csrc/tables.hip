// Hashed n-gram tables on gfx950: hash + gather-add, and the table backward with the sparse
// per-row optimizer inlined (decoder-rtx posts by Chris McCormick, baseline-4 thread: bigram
// tables added to x0 and to values, "sparse, no first moment, and only per-row magnitude",
// no .grad buffers).  The same sort + segmented reduction also produces the dense embedding
// gradient (a deterministic scatter-add without float atomics).
//
// Backward pipeline for n per-token gradient rows keyed by table row:
//   1. stable LSD radix sort of (key, token) pairs, 8-bit digits, keys outside the table
//      mapped to a sentinel that sorts last;
//   2. run boundaries -> segment starts (one segment per distinct row);
//   3. each segment is cut into chunks of SEG_CHUNK tokens; one wavefront sums one chunk in
//      ascending token order;
//   4. single-chunk segments finalize at once; longer ones write fp32 partials that a second
//      kernel adds in chunk order before finalizing.
// Summation order is fixed, so results are bitwise reproducible run to run.
#include "kernels.h"

namespace gpt {

namespace {

constexpr int SCAN_THREADS = 256, SCAN_ITEMS = 8, SCAN_TILE = SCAN_THREADS * SCAN_ITEMS;
constexpr int RS_THREADS = 256, RS_ROUNDS = 8, RS_TILE = RS_THREADS * RS_ROUNDS;
constexpr int SEG_CHUNK = 32;
constexpr uint64_t HASH_MULT = 1000003ull;

// ------------------------------------------------------------------ hash + gather
__device__ __forceinline__ uint64_t mod_rows(uint64_t x, uint64_t rows, bool pow2) {
  return pow2 ? (x & (rows - 1)) : (x % rows);
}

template <typename T>
__global__ void bigram_gather_kernel(const int32_t* __restrict__ tokens, int T_, int order,
                                     uint32_t vocab, const T* __restrict__ table,
                                     uint64_t rows, int dim, T* __restrict__ y,
                                     int32_t* __restrict__ h_out, long long n) {
  const int groups = dim / 8;
  const long long gid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n * groups) return;
  const long long tok = gid / groups;
  const int g = (int)(gid % groups);
  const int t = (int)(tok % T_);
  const bool pow2 = (rows & (rows - 1)) == 0;
  const uint64_t c = (uint32_t)tokens[tok];
  const uint64_t p = t >= 1 ? (uint64_t)(uint32_t)tokens[tok - 1] : vocab;
  uint64_t h;
  if (order == 2) {
    h = mod_rows(p * HASH_MULT + c, rows, pow2);
  } else {
    const uint64_t pp = t >= 2 ? (uint64_t)(uint32_t)tokens[tok - 2] : vocab;
    // ((pp*M + p)*M + c) mod R, reduced after the first step so nothing overflows 64 bits.
    const uint64_t a = mod_rows(pp * HASH_MULT + p, rows, pow2);
    h = mod_rows(a * HASH_MULT + c, rows, pow2);
  }
  if (h_out && g == 0) h_out[tok] = (int32_t)h;
  float a[8], b[8];
  load8_f32(y + tok * dim + g * 8, a);
  load8_f32(table + h * (uint64_t)dim + g * 8, b);
#pragma unroll
  for (int i = 0; i < 8; ++i) a[i] += b[i];
  store8_f32(y + tok * dim + g * 8, a);
}

// ------------------------------------------------------------------ exclusive scan
// Items come from a functor item(i) -> int for i in [0, n); out[i] = sum of items < i.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x % WAVE;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    int y = __shfl_up(x, o, WAVE);
    if (lane >= o) x += y;
  }
  return x;
}

// Exclusive scan of one value per thread over the block; returns the block total in *total.
__device__ __forceinline__ int block_excl_scan(int x, int* smem /* >= 16 */, int* total) {
  const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE, nw = blockDim.x / WAVE;
  int inc = wave_incl_scan(x);
  __syncthreads();
  if (lane == WAVE - 1) smem[w] = inc;
  __syncthreads();
  int before = 0, all = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < w) before += smem[i];
    all += smem[i];
  }
  *total = all;
  return before + inc - x;
}

struct ItemArray {
  const int* a;
  long long n;
  __device__ int operator()(long long i) const { return i < n ? a[i] : 0; }
};
// 1 at the first element of every run of equal sorted keys.
struct ItemRunHead {
  const uint32_t* k;
  long long n;
  __device__ int operator()(long long i) const {
    return i < n && (i == 0 || k[i] != k[i - 1]) ? 1 : 0;
  }
};
// Chunks of segment u (0 for u >= number of segments).
struct ItemChunks {
  const int* seg_start;
  const int* n_seg;
  __device__ int operator()(long long u) const {
    if (u >= *n_seg) return 0;
    int len = seg_start[u + 1] - seg_start[u];
    return (len + SEG_CHUNK - 1) / SEG_CHUNK;
  }
};
// Partial slots of segment u: its chunk count when it has more than one chunk.
struct ItemPartials {
  const int* chunk_base;
  const int* n_seg;
  __device__ int operator()(long long u) const {
    if (u >= *n_seg) return 0;
    int c = chunk_base[u + 1] - chunk_base[u];
    return c > 1 ? c : 0;
  }
};

template <class Item>
__global__ void scan_tile_sums(Item item, long long n, int* bsum) {
  __shared__ int smem[16];
  const long long base = (long long)blockIdx.x * SCAN_TILE + threadIdx.x * SCAN_ITEMS;
  int s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) s += item(base + i);
  int total;
  block_excl_scan(s, smem, &total);
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

__global__ void scan_block_sums(int* bsum, int nb, int* total_out) {
  __shared__ int smem[16];
  const int per = (nb + blockDim.x - 1) / blockDim.x;
  const int b0 = threadIdx.x * per;
  int s = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < nb) s += bsum[b0 + i];
  int total;
  int run = block_excl_scan(s, smem, &total);
  for (int i = 0; i < per; ++i)
    if (b0 + i < nb) {
      int v = bsum[b0 + i];
      bsum[b0 + i] = run;
      run += v;
    }
  if (threadIdx.x == 0 && total_out) *total_out = total;
}

template <class Item>
__global__ void scan_apply(Item item, long long n, const int* bsum, int* out) {
  __shared__ int smem[16];
  const long long base = (long long)blockIdx.x * SCAN_TILE + threadIdx.x * SCAN_ITEMS;
  int v[SCAN_ITEMS], s = 0;
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) {
    v[i] = item(base + i);
    s += v[i];
  }
  int total;
  int run = block_excl_scan(s, smem, &total) + bsum[blockIdx.x];
#pragma unroll
  for (int i = 0; i < SCAN_ITEMS; ++i) {
    if (base + i < n) out[base + i] = run;
    run += v[i];
  }
}

struct ScanScratch {
  int* bsum;  // cdiv(n, SCAN_TILE) ints
};

template <class Item>
void excl_scan(Item item, long long n, int* out, int* total, int* bsum, hipStream_t s) {
  const unsigned nb = cdiv(n, SCAN_TILE);
  scan_tile_sums<<<nb, SCAN_THREADS, 0, s>>>(item, n, bsum);
  scan_block_sums<<<1, 1024, 0, s>>>(bsum, (int)nb, total);
  scan_apply<<<nb, SCAN_THREADS, 0, s>>>(item, n, bsum, out);
}

// ------------------------------------------------------------------ radix sort
__global__ void sort_init(const int32_t* __restrict__ h, long long n, long long rows,
                          uint32_t* __restrict__ keys, uint32_t* __restrict__ vals) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t k = h[i];
  keys[i] = (k >= 0 && k < rows) ? (uint32_t)k : (uint32_t)rows;  // sentinel sorts last
  vals[i] = (uint32_t)i;
}

__global__ void radix_hist(const uint32_t* __restrict__ keys, long long n, int shift, int nblk,
                           int* __restrict__ hist /* [256][nblk] */) {
  __shared__ int cnt[256];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const long long base = (long long)blockIdx.x * RS_TILE;
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; ++r) {
    long long i = base + r * RS_THREADS + threadIdx.x;
    if (i < n) atomicAdd(&cnt[(keys[i] >> shift) & 255u], 1);
  }
  __syncthreads();
  hist[threadIdx.x * nblk + blockIdx.x] = cnt[threadIdx.x];
}

// Stable scatter: items of a tile are ranked in index order, round by round; inside a round
// lanes with equal digits are matched with 8 ballots.
__global__ void radix_scatter(const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin,
                              uint32_t* __restrict__ kout, uint32_t* __restrict__ vout,
                              long long n, int shift, int nblk, const int* __restrict__ offs) {
  __shared__ int base[256];
  __shared__ int wcnt[RS_THREADS / WAVE][256];
  const int tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
  base[tid] = offs[tid * nblk + blockIdx.x];
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r = 0; r < RS_ROUNDS; ++r) {
#pragma unroll
    for (int q = 0; q < RS_THREADS / WAVE; ++q) wcnt[q][tid] = 0;
    __syncthreads();
    const long long i = (long long)blockIdx.x * RS_TILE + r * RS_THREADS + tid;
    const bool valid = i < n;
    uint32_t k = 0, v = 0, d = 0;
    if (valid) {
      k = kin[i];
      v = vin[i];
      d = (k >> shift) & 255u;
    }
    uint64_t mask = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (d >> b) & 1u;
      const uint64_t bal = __ballot(valid && bit);
      mask &= bit ? bal : ~bal;
    }
    const int rank = __popcll(mask & lt);
    if (valid && rank == 0) wcnt[w][d] = __popcll(mask);
    __syncthreads();
    if (valid) {
      int pos = base[d] + rank;
      for (int q = 0; q < w; ++q) pos += wcnt[q][d];
      kout[pos] = k;
      vout[pos] = v;
    }
    __syncthreads();
    int add = 0;
#pragma unroll
    for (int q = 0; q < RS_THREADS / WAVE; ++q) add += wcnt[q][tid];
    base[tid] += add;
    __syncthreads();
  }
}

// ------------------------------------------------------------------ segments
__global__ void seg_scatter_starts(const uint32_t* __restrict__ k, long long n,
                                   const int* __restrict__ pos, const int* __restrict__ n_seg,
                                   int* __restrict__ seg_start) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n && (i == 0 || k[i] != k[i - 1])) seg_start[pos[i]] = (int)i;
  if (i == 0) seg_start[*n_seg] = (int)n;
}

__global__ void chunk_list(const int* __restrict__ chunk_base, const int* __restrict__ n_seg,
                           int* __restrict__ chunk_seg) {
  const long long u = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= *n_seg) return;
  for (int c = chunk_base[u]; c < chunk_base[u + 1]; ++c) chunk_seg[c] = (int)u;
}

enum { MODE_UPDATE = 0, MODE_GRAD = 1 };

template <typename T>
struct Finish {
  T* table;          // MODE_UPDATE: [rows, dim] in T
  float* v;          // MODE_UPDATE: [rows]
  float* out;        // MODE_GRAD: [rows, dim] fp32
  float lr, beta2, eps;
  int beta;
};

// acc[gi][e] holds columns (lane + 64*gi)*8 + e of the row sum g.
template <typename T, int MODE, int MAXG>
__device__ __forceinline__ void finish_row(const Finish<T>& f, uint32_t row, int dim,
                                           float (&acc)[MAXG][8]) {
  const int lane = threadIdx.x % WAVE, groups = dim / 8;
  if (MODE == MODE_GRAD) {
#pragma unroll
    for (int gi = 0; gi < MAXG; ++gi) {
      const int g = lane + gi * WAVE;
      if (g < groups) {
        float* o = f.out + (size_t)row * dim + g * 8;
        float r[8];
        if (f.beta) {
          f32x8 old = *reinterpret_cast<const f32x8*>(o);
#pragma unroll
          for (int e = 0; e < 8; ++e) r[e] = old[e] + acc[gi][e];
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) r[e] = acc[gi][e];
        }
        store8_f32(o, r);
      }
    }
  } else {
    float ss = 0.f;
#pragma unroll
    for (int gi = 0; gi < MAXG; ++gi)
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += acc[gi][e] * acc[gi][e];
    ss = wave_sum(ss);
    const float vr = f.beta2 * f.v[row] + (1.f - f.beta2) * (ss / (float)dim);
    const float step = f.lr / (sqrtf(vr) + f.eps);
    if (lane == 0) f.v[row] = vr;
#pragma unroll
    for (int gi = 0; gi < MAXG; ++gi) {
      const int g = lane + gi * WAVE;
      if (g < groups) {
        T* p = f.table + (size_t)row * dim + g * 8;
        float w[8];
        load8_f32(p, w);
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] -= step * acc[gi][e];
        store8_f32(p, w);
      }
    }
  }
}

template <typename T, typename DyT, int MODE, int MAXG>
__global__ __launch_bounds__(256) void seg_chunk_kernel(
    const uint32_t* __restrict__ skeys, const uint32_t* __restrict__ svals,
    const DyT* __restrict__ dy, int dim, long long rows, const int* __restrict__ seg_start,
    const int* __restrict__ chunk_base, const int* __restrict__ chunk_seg,
    const int* __restrict__ n_chunks, const int* __restrict__ pbase, float* __restrict__ partial,
    Finish<T> fin) {
  const int lane = threadIdx.x % WAVE, groups = dim / 8;
  const int wpb = blockDim.x / WAVE;
  const int total = *n_chunks;
  for (int c = blockIdx.x * wpb + threadIdx.x / WAVE; c < total; c += gridDim.x * wpb) {
    const int u = chunk_seg[c];
    const int s0 = seg_start[u], s1 = seg_start[u + 1];
    const uint32_t row = skeys[s0];
    if (row >= rows) continue;  // out-of-range keys (sentinel) are skipped
    const int nch = chunk_base[u + 1] - chunk_base[u];
    const int j = c - chunk_base[u];
    const int a = s0 + j * SEG_CHUNK, b = min(a + SEG_CHUNK, s1);
    float acc[MAXG][8];
#pragma unroll
    for (int gi = 0; gi < MAXG; ++gi)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[gi][e] = 0.f;
    for (int i = a; i < b; ++i) {
      const size_t t = svals[i];
#pragma unroll
      for (int gi = 0; gi < MAXG; ++gi) {
        const int g = lane + gi * WAVE;
        if (g < groups) {
          float x[8];
          load8_f32(dy + t * dim + g * 8, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[gi][e] += x[e];
        }
      }
    }
    if (nch == 1) {
      finish_row<T, MODE, MAXG>(fin, row, dim, acc);
    } else {
      float* p = partial + (size_t)(pbase[u] + j) * dim;
#pragma unroll
      for (int gi = 0; gi < MAXG; ++gi) {
        const int g = lane + gi * WAVE;
        if (g < groups) store8_f32(p + g * 8, acc[gi]);
      }
    }
  }
}

template <typename T, int MODE, int MAXG>
__global__ __launch_bounds__(256) void seg_finish_kernel(
    const uint32_t* __restrict__ skeys, int dim, long long rows,
    const int* __restrict__ seg_start, const int* __restrict__ chunk_base,
    const int* __restrict__ n_seg, const int* __restrict__ pbase,
    const float* __restrict__ partial, Finish<T> fin) {
  const int lane = threadIdx.x % WAVE, groups = dim / 8;
  const int wpb = blockDim.x / WAVE;
  const int total = *n_seg;
  for (int u = blockIdx.x * wpb + threadIdx.x / WAVE; u < total; u += gridDim.x * wpb) {
    const int nch = chunk_base[u + 1] - chunk_base[u];
    if (nch <= 1) continue;
    const uint32_t row = skeys[seg_start[u]];
    if (row >= rows) continue;
    float acc[MAXG][8];
#pragma unroll
    for (int gi = 0; gi < MAXG; ++gi)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[gi][e] = 0.f;
    for (int j = 0; j < nch; ++j) {
      const float* p = partial + (size_t)(pbase[u] + j) * dim;
#pragma unroll
      for (int gi = 0; gi < MAXG; ++gi) {
        const int g = lane + gi * WAVE;
        if (g < groups) {
          float x[8];
          load8_f32(p + g * 8, x);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[gi][e] += x[e];
        }
      }
    }
    finish_row<T, MODE, MAXG>(fin, row, dim, acc);
  }
}

// Workspace carve for n keys of width dim.
struct SegWs {
  uint32_t *k0, *k1, *v0, *v1;
  int *hist, *bsum, *pos, *seg_start, *chunk_base, *chunk_seg, *pbase, *counters;
  float* partial;
};

SegWs carve_seg(Carver& c, long long n, int dim) {
  SegWs w;
  const long long nblk = cdiv(n, RS_TILE);
  const long long max_chunks = n + n / SEG_CHUNK + 1;
  const long long max_partials = 2 * (n / SEG_CHUNK) + 2;
  w.k0 = c.take<uint32_t>(n);
  w.k1 = c.take<uint32_t>(n);
  w.v0 = c.take<uint32_t>(n);
  w.v1 = c.take<uint32_t>(n);
  w.hist = c.take<int>(256 * nblk);
  w.bsum = c.take<int>(cdiv(std::max<long long>(256 * nblk, n + 1), SCAN_TILE) + 1);
  w.pos = c.take<int>(std::max<long long>(256 * nblk, n + 1));
  w.seg_start = c.take<int>(n + 2);
  w.chunk_base = c.take<int>(n + 2);
  w.chunk_seg = c.take<int>(max_chunks);
  w.pbase = c.take<int>(n + 2);
  w.counters = c.take<int>(8);
  w.partial = c.take<float>((size_t)max_partials * dim);
  return w;
}

template <typename T, typename DyT, int MODE>
gpt_status segsum_run(const int32_t* keys, const DyT* dy, long long n, int dim, long long rows,
                      Finish<T> fin, void* ws, size_t ws_bytes, hipStream_t s) {
  if (n == 0) return GPT_OK;
  Carver c(ws, ws_bytes);
  SegWs w = carve_seg(c, n, dim);
  if (!c.ok) return fail(GPT_EWORKSPACE, "segment workspace too small");
  int* n_seg = w.counters + 0;
  int* n_chunks = w.counters + 1;
  int* n_partials = w.counters + 2;
  const int nblk = (int)cdiv(n, RS_TILE);

  sort_init<<<cdiv(n, 256), 256, 0, s>>>(keys, n, rows, w.k0, w.v0);
  int bits = 1;
  while (bits < 32 && ((uint64_t)rows >> bits) != 0) ++bits;  // sentinel `rows` must fit
  uint32_t *ki = w.k0, *vi = w.v0, *ko = w.k1, *vo = w.v1;
  for (int shift = 0; shift < bits; shift += 8) {
    radix_hist<<<nblk, RS_THREADS, 0, s>>>(ki, n, shift, nblk, w.hist);
    excl_scan(ItemArray{w.hist, 256LL * nblk}, 256LL * nblk, w.pos, nullptr, w.bsum, s);
    radix_scatter<<<nblk, RS_THREADS, 0, s>>>(ki, vi, ko, vo, n, shift, nblk, w.pos);
    std::swap(ki, ko);
    std::swap(vi, vo);
  }
  // segments
  excl_scan(ItemRunHead{ki, n}, n, w.pos, n_seg, w.bsum, s);
  seg_scatter_starts<<<cdiv(n, 256), 256, 0, s>>>(ki, n, w.pos, n_seg, w.seg_start);
  excl_scan(ItemChunks{w.seg_start, n_seg}, n + 1, w.chunk_base, n_chunks, w.bsum, s);
  chunk_list<<<cdiv(n, 256), 256, 0, s>>>(w.chunk_base, n_seg, w.chunk_seg);
  excl_scan(ItemPartials{w.chunk_base, n_seg}, n + 1, w.pbase, n_partials, w.bsum, s);

  const unsigned grid = (unsigned)std::min<long long>(cdiv(n, 4), 8192);
  const int maxg = (dim / 8 + WAVE - 1) / WAVE;
#define SEG_LAUNCH(G)                                                                          \
  do {                                                                                         \
    seg_chunk_kernel<T, DyT, MODE, G><<<grid, 256, 0, s>>>(ki, vi, dy, dim, rows, w.seg_start, \
                                                           w.chunk_base, w.chunk_seg, n_chunks, \
                                                           w.pbase, w.partial, fin);           \
    seg_finish_kernel<T, MODE, G><<<grid, 256, 0, s>>>(ki, dim, rows, w.seg_start,              \
                                                       w.chunk_base, n_seg, w.pbase,            \
                                                       w.partial, fin);                         \
  } while (0)
  switch (maxg) {
    case 1: SEG_LAUNCH(1); break;
    case 2: SEG_LAUNCH(2); break;
    case 3: SEG_LAUNCH(3); break;
    case 4: SEG_LAUNCH(4); break;
    default: return fail(GPT_ESHAPE, "row width above 2048 is not supported");
  }
#undef SEG_LAUNCH
  return check_launch("segment reduce");
}

}  // namespace

size_t segsum_workspace_bytes(long long n, int dim) {
  Carver c(nullptr, 0);
  carve_seg(c, std::max<long long>(n, 1), dim);
  return c.size();
}

template <typename T>
gpt_status launch_bigram_fwd(const int32_t* tokens, int B, int T_, int order, int vocab,
                             const T* table, long long rows, int dim, T* y, int32_t* h_out,
                             hipStream_t s) {
  const long long n = (long long)B * T_;
  if (n == 0) return GPT_OK;
  const long long threads = n * (dim / 8);
  bigram_gather_kernel<T><<<cdiv(threads, 256), 256, 0, s>>>(
      tokens, T_, order, (uint32_t)vocab, table, (uint64_t)rows, dim, y, h_out, n);
  return check_launch("bigram_fwd");
}

template <typename T>
gpt_status segsum_update(const int32_t* keys, const T* dy, long long n, int dim, T* table,
                         float* v, long long rows, float lr, float beta2, float eps, void* ws,
                         size_t ws_bytes, hipStream_t s) {
  Finish<T> fin{table, v, nullptr, lr, beta2, eps, 0};
  return segsum_run<T, T, MODE_UPDATE>(keys, dy, n, dim, rows, fin, ws, ws_bytes, s);
}

gpt_status segsum_grad(const int32_t* keys, const float* dy, long long n, int dim, float* out,
                       long long rows, int beta, void* ws, size_t ws_bytes, hipStream_t s) {
  Finish<float> fin{nullptr, nullptr, out, 0.f, 0.f, 0.f, beta};
  return segsum_run<float, float, MODE_GRAD>(keys, dy, n, dim, rows, fin, ws, ws_bytes, s);
}

template gpt_status launch_bigram_fwd<float>(const int32_t*, int, int, int, int, const float*,
                                             long long, int, float*, int32_t*, hipStream_t);
template gpt_status launch_bigram_fwd<bf16>(const int32_t*, int, int, int, int, const bf16*,
                                            long long, int, bf16*, int32_t*, hipStream_t);
template gpt_status segsum_update<float>(const int32_t*, const float*, long long, int, float*,
                                         float*, long long, float, float, float, void*, size_t,
                                         hipStream_t);
template gpt_status segsum_update<bf16>(const int32_t*, const bf16*, long long, int, bf16*,
                                        float*, long long, float, float, float, void*, size_t,
                                        hipStream_t);

}  // namespace gpt
