// Hashed n-gram tables on gfx950: hash + gather-add, and the table backward with the sparse
// per-row optimizer inlined (ChrisJMcCormick post feed, the posts on the hashed bigram tables
// added to x0 and to the attention values: the table optimizer keeps no momentum and one
// magnitude statistic per row, and no gradient buffer exists).  The same sort + segmented
// reduction also produces the dense embedding gradient (a deterministic scatter-add without
// float atomics).
//
// Backward pipeline for n per-token gradient rows keyed by table row:
//   1. stable LSD radix sort of (key, token) pairs, 8-bit digits, keys outside the table
//      mapped to a sentinel that sorts last: per pass a tile histogram and a scatter that
//      scans the histogram for its own offsets;
//   2. one wavefront per tile of SEG_TILE sorted positions sums the runs of equal keys it
//      holds in ascending sorted (= token) order and finalizes the rows that lie inside it;
//   3. rows crossing tile edges leave fp32 partials that a second kernel adds in tile order
//      before finalizing.
// Summation order is fixed, so results are bitwise reproducible run to run.
#include "kernels.h"

namespace gpt {

namespace {

constexpr int RS_THREADS = 256, RS_ROUNDS = 8, RS_TILE = RS_THREADS * RS_ROUNDS;
constexpr int SEG_TILE = 64;  // sorted positions per wavefront in the segmented sums
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

// ------------------------------------------------------------------ radix sort
constexpr int INLINE_OFFS_TILES = 256;  // up to this many tiles the scatter finds its own offsets

__device__ __forceinline__ uint32_t clamp_key(int32_t k, long long rows) {
  return (k >= 0 && k < rows) ? (uint32_t)k : (uint32_t)rows;  // sentinel sorts last
}

// hist[d][blk] = number of keys of tile blk (current order) whose digit at `shift` is d.  The
// first pass reads the keys straight from h.
__global__ void radix_hist(const int32_t* __restrict__ h, const uint32_t* __restrict__ keys,
                           long long n, long long rows, int shift, int nblk,
                           int* __restrict__ hist) {
  __shared__ int cnt[256];
  cnt[threadIdx.x] = 0;
  __syncthreads();
  const long long base = (long long)blockIdx.x * RS_TILE;
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; ++r) {
    const long long i = base + r * RS_THREADS + threadIdx.x;
    if (i < n) {
      const uint32_t k = h ? clamp_key(h[i], rows) : keys[i];
      atomicAdd(&cnt[(k >> shift) & 255u], 1);
    }
  }
  __syncthreads();
  hist[(long long)threadIdx.x * nblk + blockIdx.x] = cnt[threadIdx.x];
}

// Scatter offset of digit d in tile blk: all keys of smaller digits plus digit d's keys in
// earlier tiles (exclusive scan of hist in [digit][tile] order).
// The digit's row of tile counts is read 64 counts per round trip (16-byte loads, all issued
// before any is used) when its length allows it.
__device__ __forceinline__ int digit_offset(const int* __restrict__ hist, int nblk, int* smem) {
  const int d = threadIdx.x;
  const int* row = hist + (long long)d * nblk;
  const int me = (int)blockIdx.x;
  int before = 0, total = 0;
  if (nblk % 4 == 0) {  // rows of 16-byte groups (the workspace is 256-byte aligned)
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const i32x4* row4 = reinterpret_cast<const i32x4*>(row);
    const int n4 = nblk / 4;
    for (int c0 = 0; c0 < n4; c0 += 16) {
      i32x4 v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = c0 + i < n4 ? row4[c0 + i] : i32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          total += v[i][e];
          before += 4 * (c0 + i) + e < me ? v[i][e] : 0;
        }
    }
  } else {
#pragma unroll 8
    for (int b = 0; b < nblk; ++b) {
      const int c = row[b];
      total += c;
      before += (b < me) ? c : 0;
    }
  }
  int all;
  return block_excl_scan(total, smem, &all) + before;
}

// Offsets for many tiles: the same scan by one workgroup, written to hist in place.
__global__ __launch_bounds__(1024) void radix_offsets(int* __restrict__ a, int nblk) {
  __shared__ int smem[16];
  const long long m = 256LL * nblk;
  const long long per = (m + blockDim.x - 1) / blockDim.x;
  const long long b0 = (long long)threadIdx.x * per;
  int s = 0;
  for (long long i = 0; i < per; ++i)
    if (b0 + i < m) s += a[b0 + i];
  int total;
  int run = block_excl_scan(s, smem, &total);
  for (long long i = 0; i < per; ++i)
    if (b0 + i < m) {
      const int v = a[b0 + i];
      a[b0 + i] = run;
      run += v;
    }
}

// Stable scatter of one digit: items of a tile are ranked in index order, round by round;
// inside a round lanes with equal digits are matched with 8 ballots.  The first pass reads
// the keys from h (clamped) with values = token index.  `scanned`: hist already holds offsets.
__global__ void radix_scatter(const int32_t* __restrict__ h, long long rows,
                              const uint32_t* __restrict__ kin, const uint32_t* __restrict__ vin,
                              uint32_t* __restrict__ kout, uint32_t* __restrict__ vout,
                              long long n, int shift, int nblk, const int* __restrict__ hist,
                              int scanned) {
  __shared__ int base[256];
  __shared__ int wcnt[RS_THREADS / WAVE][256];
  __shared__ int smem[16];
  const int tid = threadIdx.x, lane = tid % WAVE, w = tid / WAVE;
  // every round's key and value are loaded up front (one memory round trip for the tile, in
  // flight while the digit offsets are formed)
  uint32_t kr[RS_ROUNDS], vr[RS_ROUNDS];
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; ++r) {
    const long long i = (long long)blockIdx.x * RS_TILE + r * RS_THREADS + tid;
    kr[r] = 0;
    vr[r] = 0;
    if (i < n) {
      if (h) {
        kr[r] = clamp_key(h[i], rows);
        vr[r] = (uint32_t)i;
      } else {
        kr[r] = kin[i];
        vr[r] = vin[i];
      }
    }
  }
  base[tid] = scanned ? hist[(long long)tid * nblk + blockIdx.x] : digit_offset(hist, nblk, smem);
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
  for (int r = 0; r < RS_ROUNDS; ++r) {
#pragma unroll
    for (int q = 0; q < RS_THREADS / WAVE; ++q) wcnt[q][tid] = 0;
    __syncthreads();
    const long long i = (long long)blockIdx.x * RS_TILE + r * RS_THREADS + tid;
    const bool valid = i < n;
    const uint32_t k = kr[r], v = vr[r];
    const uint32_t d = valid ? (k >> shift) & 255u : 0u;
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

// ------------------------------------------------------------------ per-row sums + finish
enum { MODE_UPDATE = 0, MODE_GRAD = 1 };

template <typename T>
struct Finish {
  T* table;          // MODE_UPDATE: [rows, dim] in T
  float* v;          // MODE_UPDATE: [rows]
  float* out;        // MODE_GRAD: [rows, dim] fp32
  float lr, beta2, eps;
  int beta;
};

// Rows are moved through a buffer resource over the one row (its base is wave-uniform), lane l
// owning the 4-element groups q = l + 64*gi (gi < G), columns 4q .. 4q+3.  Lanes past the row's
// end get an offset beyond the resource: their loads read zeros and their stores are dropped,
// so no load or store sits behind a per-lane branch.
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr uint32_t ROW_OOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, bytes, 0x00020000);
}

// Raw words of four elements (bf16: two dwords, fp32: four) and their float values.
template <typename S> struct Raw4;
template <> struct Raw4<bf16> {
  typedef u32x2 type;
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b64(rs, off * 2, 0, 0);
  }
  static __device__ __forceinline__ void cvt(type v, float (&o)[4]) {
    o[0] = __uint_as_float(v[0] << 16);
    o[1] = __uint_as_float(v[0] & 0xffff0000u);
    o[2] = __uint_as_float(v[1] << 16);
    o[3] = __uint_as_float(v[1] & 0xffff0000u);
  }
};
template <> struct Raw4<float> {
  typedef u32x4 type;
  static __device__ __forceinline__ type load(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(rs, off * 4, 0, 0);
  }
  static __device__ __forceinline__ void cvt(type v, float (&o)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(v[e]);
  }
};
template <typename S>
__device__ __forceinline__ void ld4(__amdgpu_buffer_rsrc_t rs, uint32_t off, const S*, float (&o)[4]) {
  Raw4<S>::cvt(Raw4<S>::load(rs, off), o);
}
__device__ __forceinline__ void st4(__amdgpu_buffer_rsrc_t rs, uint32_t off, bf16*, const float (&o)[4]) {
  bf16x4 b;
#pragma unroll
  for (int e = 0; e < 4; ++e) b[e] = (bf16)o[e];
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, b), rs, off * 2, 0, 0);
}
__device__ __forceinline__ void st4(__amdgpu_buffer_rsrc_t rs, uint32_t off, float*, const float (&o)[4]) {
  const u32x4 v = {__float_as_uint(o[0]), __float_as_uint(o[1]), __float_as_uint(o[2]),
                   __float_as_uint(o[3])};
  __builtin_amdgcn_raw_buffer_store_b128(v, rs, off * 4, 0, 0);
}

template <int G>
__device__ __forceinline__ void zero_acc(float (&a)[G][4]) {
#pragma unroll
  for (int gi = 0; gi < G; ++gi)
#pragma unroll
    for (int e = 0; e < 4; ++e) a[gi][e] = 0.f;
}

// element offset of lane's group gi, or past the end (elements; scaled to bytes in ld4/st4)
__device__ __forceinline__ uint32_t group_off(int gi, int dim) {
  const int q = threadIdx.x % WAVE + gi * WAVE;
  return q * 4 < dim ? (uint32_t)(q * 4) : ROW_OOB / 4;
}

// live == false (wave-uniform): every lane reads zeros.
template <int G, typename S>
__device__ __forceinline__ void load_row(const S* p, int dim, float (&x)[G][4], bool live = true) {
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(p, dim * (int)sizeof(S));
#pragma unroll
  for (int gi = 0; gi < G; ++gi) ld4(rs, live ? group_off(gi, dim) : ROW_OOB / 4, p, x[gi]);
}

template <int G, typename S>
__device__ __forceinline__ void store_row(S* p, int dim, const float (&x)[G][4]) {
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(p, dim * (int)sizeof(S));
#pragma unroll
  for (int gi = 0; gi < G; ++gi) st4(rs, group_off(gi, dim), p, x[gi]);
}

// What the row's finish reads, fetched before the sums so that both latencies overlap (kept as
// raw words until the finish, so nothing waits for them earlier).
template <typename T, int MODE, int G>
struct FinishIn {
  using S = typename std::conditional<MODE == MODE_UPDATE, T, float>::type;
  typename Raw4<S>::type raw[G];  // MODE_UPDATE: table row; MODE_GRAD: old output row
  float v;                        // MODE_UPDATE: second moment of the row
  bool have;                      // MODE_GRAD: beta = 1 (old output row loaded)
  __device__ __forceinline__ void fetch(const Finish<T>& f, uint32_t row, int stride, int width) {
    const S* p;
    if constexpr (MODE == MODE_UPDATE) {
      v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(row_rsrc(f.v + row, 4), 0, 0, 0));
      p = f.table + (size_t)row * stride;
      have = true;
    } else {
      v = 0.f;
      p = f.out + (size_t)row * stride;
      have = f.beta != 0;
    }
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(p, width * (int)sizeof(S));
#pragma unroll
    for (int gi = 0; gi < G; ++gi) raw[gi] = Raw4<S>::load(rs, have ? group_off(gi, width) : ROW_OOB / 4);
  }
  __device__ __forceinline__ void values(float (&w)[G][4]) const {
#pragma unroll
    for (int gi = 0; gi < G; ++gi) Raw4<S>::cvt(raw[gi], w[gi]);
  }
};

// MODE_UPDATE: v = beta2 v + (1 - beta2) mean(g^2); w -= lr g / (sqrt(v) + eps).
// MODE_GRAD: out = (beta ? out : 0) + g.
// Row `row` of `stride` elements, of which this wave owns `width` (MODE_UPDATE: the whole row,
// since its statistic needs every element; MODE_GRAD: one column slice, pointers pre-offset).
template <typename T, int MODE, int G>
__device__ __forceinline__ void finish_row(const Finish<T>& f, uint32_t row, int stride, int width,
                                           const float (&acc)[G][4], const FinishIn<T, MODE, G>& in) {
  float w[G][4];
  in.values(w);
  if constexpr (MODE == MODE_GRAD) {
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int e = 0; e < 4; ++e) w[gi][e] += acc[gi][e];
    store_row<G>(f.out + (size_t)row * stride, width, w);
  } else {
    const int dim = width;
    float ss = 0.f;
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int e = 0; e < 4; ++e) ss += acc[gi][e] * acc[gi][e];
    ss = wave_sum(ss);
    const float vr = f.beta2 * in.v + (1.f - f.beta2) * (ss / (float)dim);
    const float step = f.lr / (sqrtf(vr) + f.eps);
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
      for (int e = 0; e < 4; ++e) w[gi][e] -= step * acc[gi][e];
    store_row<G>(f.table + (size_t)row * stride, dim, w);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vr), row_rsrc(f.v + row, 4),
                                          threadIdx.x % WAVE == 0 ? 0u : ROW_OOB, 0, 0);
  }
}

// Rows in flight per wave while summing (register budget: U * G * 4 floats).
template <int G> constexpr int unroll_rows() { return G <= 1 ? 8 : (G <= 2 ? 4 : 2); }

constexpr uint32_t NO_KEY = 0xffffffffu;  // above every key (keys <= rows < 2^31)

// Sum of the gradient rows of sorted positions [j, pe) of the tile (token ids in `tok`,
// lane-indexed), in ascending order with U rows in flight.  Slots past pe load zeros, which
// leave the sum unchanged, so the U loads of a round are issued back to back.
template <int G, int U, typename DyT>
__device__ __forceinline__ void sum_rows(const DyT* __restrict__ dy, int stride, int width,
                                         uint32_t tok, int j, int pe, float (&acc)[G][4]) {
  zero_acc<G>(acc);
  for (int j0 = j; j0 < pe; j0 += U) {
    float x[U][G][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t t = (uint32_t)__builtin_amdgcn_readlane((int)tok, min(j0 + u, pe - 1));
      load_row<G>(dy + t * stride, width, x[u], j0 + u < pe);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[gi][q] += x[u][gi][q];
  }
}

// A run of equal keys inside one tile ("piece"): sorted positions [j, pe) of the tile.
struct Piece {
  int j, pe;
  uint32_t row;
  bool live, starts, ends;  // live: row inside the table
};

// Loads of one piece, issued ahead of the previous piece's stores and kept as raw words: the
// finish operands and the first U gradient rows.  A piece that is not live loads zeros.
template <typename T, typename DyT, int MODE, int G, int U>
struct PieceLoads {
  FinishIn<T, MODE, G> in;
  typename Raw4<DyT>::type x[U][G];
  __device__ __forceinline__ void issue(const Piece& p, const DyT* __restrict__ dy, int stride,
                                        int width, uint32_t tok, const Finish<T>& fin) {
    in.fetch(fin, p.live ? p.row : 0u, stride, width);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool on = p.live && p.j + u < p.pe;
      const size_t t = (uint32_t)__builtin_amdgcn_readlane((int)tok, min(p.j + u, p.pe - 1));
      const DyT* r = dy + t * stride;
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(r, width * (int)sizeof(DyT));
#pragma unroll
      for (int gi = 0; gi < G; ++gi) x[u][gi] = Raw4<DyT>::load(rs, on ? group_off(gi, width) : ROW_OOB / 4);
    }
  }
  // the piece's gradient sum: the rows in flight, then (long pieces) the rest
  __device__ __forceinline__ void sum(const Piece& p, const DyT* __restrict__ dy, int stride,
                                      int width, uint32_t tok, float (&acc)[G][4]) const {
    zero_acc<G>(acc);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int gi = 0; gi < G; ++gi) {
        float x4[4];
        Raw4<DyT>::cvt(x[u][gi], x4);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[gi][q] += x4[q];
      }
    if (p.j + U < p.pe) {
      float rest[G][4];
      sum_rows<G, U>(dy, stride, width, tok, p.j + U, p.pe, rest);
#pragma unroll
      for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[gi][q] += rest[gi][q];
    }
  }
};

// One wavefront per tile of SEG_TILE sorted positions: keys and token ids arrive in one load
// each, the pieces come from one ballot, and each piece's gradient rows are summed in sorted
// (= token) order.  Only a tile's first piece (continuing a row from earlier tiles) and last
// piece (a row that goes on) can be incomplete: their sums go to partial slots 2*tile and
// 2*tile + 1.  Keys past the table (the sentinel) form a suffix and are skipped.  The complete
// pieces are finished in a loop whose every pass issues the loads of the next piece, stores
// the current one and then consumes the next piece's loads, so no load wait covers a store.
// Rows have `stride` elements; blockIdx.y selects the column slice [y * sw, y * sw + sw) that
// the block's waves own (MODE_GRAD splits wide rows so that small n still fills the GPU;
// MODE_UPDATE has one slice, sw = stride, as its row statistic needs the whole row).
template <typename T, typename DyT, int MODE, int G>
__global__ __launch_bounds__(256) void seg_tile_kernel(
    const uint32_t* __restrict__ skeys, const uint32_t* __restrict__ svals,
    const DyT* __restrict__ dy, long long n, int stride, int sw, long long rows,
    float* __restrict__ partial, Finish<T> fin) {
  constexpr int U = unroll_rows<G>();
  const int col0 = blockIdx.y * sw, width = min(sw, stride - col0);
  dy += col0;
  partial += col0;
  if constexpr (MODE == MODE_GRAD) fin.out += col0;
  const int lane = threadIdx.x % WAVE;
  const int wpb = blockDim.x / WAVE;
  const long long ntiles = (n + SEG_TILE - 1) / SEG_TILE;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  for (long long tile = (long long)blockIdx.x * wpb + wave; tile < ntiles;
       tile += (long long)gridDim.x * wpb) {
    const long long P = tile * SEG_TILE;
    const int len = (int)min<long long>(SEG_TILE, n - P);
    const uint32_t key = lane < len ? skeys[P + lane] : NO_KEY;
    const uint32_t tok = lane < len ? svals[P + lane] : 0u;
    const uint32_t prevkey = P > 0 ? skeys[P - 1] : NO_KEY;
    const uint32_t nextkey = P + SEG_TILE < n ? skeys[P + SEG_TILE] : NO_KEY;
    const uint32_t left = __shfl_up(key, 1, WAVE);
    const uint64_t heads = __ballot(lane < len && (lane == 0 || key != left));
    const uint64_t dead = __ballot(lane < len && key >= rows);
    const int lim = dead ? (int)__builtin_ctzll(dead) : len;  // live positions [0, lim)
    auto piece_at = [&](int j) {
      Piece p;
      const uint64_t later = (j + 1 < WAVE) ? (heads & (~0ull << (j + 1))) : 0ull;
      p.j = j;
      p.pe = min(later ? (int)__builtin_ctzll(later) : len, lim);
      p.row = (uint32_t)__builtin_amdgcn_readlane((int)key, min(j, WAVE - 1));
      p.live = j < lim;
      p.starts = j > 0 || prevkey != p.row;
      p.ends = p.pe < len || nextkey != p.row;
      return p;
    };
    auto to_partial = [&](const Piece& p, long long slot) {
      float acc[G][4];
      sum_rows<G, U>(dy, stride, width, tok, p.j, p.pe, acc);
      store_row<G>(partial + (size_t)slot * stride, width, acc);
    };
    if (lim == 0) continue;
    int a = 0, b = lim;  // the complete pieces cover positions [a, b)
    {
      const Piece p = piece_at(0);
      if (!p.starts) {
        to_partial(p, 2 * tile);
        a = p.pe;
      }
    }
    if (a < b && lim == len) {
      const int jl = 63 - (int)__builtin_clzll(heads);
      const Piece p = piece_at(jl);
      if (!p.ends && jl >= a) {
        to_partial(p, 2 * tile + 1);
        b = jl;
      }
    }
    if (a >= b) continue;
    auto clip = [&](Piece p) {
      p.pe = min(p.pe, b);
      p.live = p.j < b;
      return p;
    };
    Piece cur = clip(piece_at(a));
    PieceLoads<T, DyT, MODE, G, U> ld;
    ld.issue(cur, dy, stride, width, tok, fin);
    float acc[G][4];
    ld.sum(cur, dy, stride, width, tok, acc);
    FinishIn<T, MODE, G> in = ld.in;
    while (true) {
      // past the last piece the next one is not live: it loads and sums zeros
      const Piece nxt = clip(piece_at(min(cur.pe, WAVE - 1)));
      ld.issue(nxt, dy, stride, width, tok, fin);
      __builtin_amdgcn_sched_barrier(0);  // the next piece's loads stay ahead of these stores
      finish_row<T, MODE, G>(fin, cur.row, stride, width, acc, in);
      __builtin_amdgcn_sched_barrier(0);
      const bool last = cur.pe >= b;
      cur = nxt;
      ld.sum(cur, dy, stride, width, tok, acc);
      in = ld.in;
      if (last) break;
    }
  }
}

// One wavefront per row that starts in a tile and goes on past it (found at that tile): adds
// the row's first partial and then the partials of the following tiles, which begin with the
// row, in tile order.  Their first keys are read 64 tiles at a time.  Column slices as in
// seg_tile_kernel.
template <typename T, int MODE, int G>
__global__ __launch_bounds__(256) void seg_tile_finish_kernel(
    const uint32_t* __restrict__ skeys, long long n, int stride, int sw, long long rows,
    const float* __restrict__ partial, Finish<T> fin) {
  constexpr int U = G <= 4 ? 8 : 4;  // partial rows in flight
  const int col0 = blockIdx.y * sw, width = min(sw, stride - col0);
  partial += col0;
  if constexpr (MODE == MODE_GRAD) fin.out += col0;
  const int lane = threadIdx.x % WAVE;
  const int wpb = blockDim.x / WAVE;
  const long long ntiles = (n + SEG_TILE - 1) / SEG_TILE;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE);
  for (long long tile = (long long)blockIdx.x * wpb + wave; tile + 1 < ntiles;
       tile += (long long)gridDim.x * wpb) {
    const long long P = tile * SEG_TILE;  // not the last tile: all SEG_TILE positions exist
    const uint32_t row = skeys[P + SEG_TILE - 1];
    if (row >= rows || skeys[P + SEG_TILE] != row) continue;         // last piece ends here
    if (skeys[P] == row && P > 0 && skeys[P - 1] == row) continue;    // the row began earlier
    FinishIn<T, MODE, G> in;
    in.fetch(fin, row, stride, width);
    float acc[G][4];
    load_row<G>(partial + (size_t)(2 * tile + 1) * stride, width, acc);
    for (long long t0 = tile + 1;; t0 += WAVE) {
      const long long t = t0 + lane;
      const bool cont = t < ntiles && skeys[t * SEG_TILE] == row;  // a prefix of the lanes
      const int cnt = __popcll(__ballot(cont));
      for (int j0 = 0; j0 < cnt; j0 += U) {
        float x[U][G][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
          load_row<G>(partial + (size_t)(2 * (t0 + min(j0 + u, cnt - 1))) * stride, width, x[u],
                      j0 + u < cnt);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
          for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[gi][q] += x[u][gi][q];
      }
      if (cnt < WAVE) break;
    }
    finish_row<T, MODE, G>(fin, row, stride, width, acc, in);
  }
}

// Workspace carve for n keys of width dim.
struct SegWs {
  uint32_t *k0, *k1, *v0, *v1;
  int* hist;
  float* partial;
};

SegWs carve_seg(Carver& c, long long n, int dim) {
  SegWs w;
  const long long nblk = cdiv(n, RS_TILE);
  const long long ntiles = (n + SEG_TILE - 1) / SEG_TILE;
  w.k0 = c.take<uint32_t>(n);
  w.k1 = c.take<uint32_t>(n);
  w.v0 = c.take<uint32_t>(n);
  w.v1 = c.take<uint32_t>(n);
  w.hist = c.take<int>(256 * nblk);
  w.partial = c.take<float>((size_t)(2 * ntiles) * dim);
  return w;
}

template <typename T, typename DyT, int MODE>
gpt_status segsum_run(const int32_t* keys, const DyT* dy, long long n, int dim, long long rows,
                      Finish<T> fin, void* ws, size_t ws_bytes, hipStream_t s) {
  if (n == 0) return GPT_OK;
  Carver c(ws, ws_bytes);
  SegWs w = carve_seg(c, n, dim);
  if (!c.ok) return fail(GPT_EWORKSPACE, "segment workspace too small");
  const int nblk = (int)cdiv(n, RS_TILE);
  const bool inline_offs = nblk <= INLINE_OFFS_TILES;

  int bits = 1;
  while (bits < 32 && ((uint64_t)rows >> bits) != 0) ++bits;  // sentinel `rows` must fit
  const int passes = (bits + 7) / 8;
  uint32_t *ki = nullptr, *vi = nullptr, *ko = w.k0, *vo = w.v0;
  for (int p = 0; p < passes; ++p) {
    const int32_t* hk = p == 0 ? keys : nullptr;
    radix_hist<<<nblk, RS_THREADS, 0, s>>>(hk, ki, n, rows, 8 * p, nblk, w.hist);
    if (!inline_offs) radix_offsets<<<1, 1024, 0, s>>>(w.hist, nblk);
    radix_scatter<<<nblk, RS_THREADS, 0, s>>>(hk, rows, ki, vi, ko, vo, n, 8 * p, nblk, w.hist,
                                              inline_offs ? 0 : 1);
    ki = ko;
    vi = vo;
    ko = (ko == w.k0) ? w.k1 : w.k0;
    vo = (vo == w.v0) ? w.v1 : w.v0;
  }

  const long long ntiles = (n + SEG_TILE - 1) / SEG_TILE;
  // MODE_GRAD: rows of a multiple of 512 elements are halved into column slices (of at least
  // 256, so every lane of a wave has work) while the tiles alone give fewer than 2048 wavefronts
  // (the embedding gradient of 16,384 tokens has 256 tiles: 8 slices of a 2048-wide row give
  // 2048 wavefronts with 8 rows in flight each).  A 768-wide row stays whole: its 192-wide
  // quarters left a quarter of the lanes idle and ran slower (GPT-2-small: 45.6 -> 54 us).
  int sw = dim;
  if (MODE == MODE_GRAD)
    while (sw % 512 == 0 && ntiles * (dim / sw) < 2048) sw /= 2;
  const unsigned grid = (unsigned)std::min<long long>(cdiv(ntiles, 4), 16384);
  const dim3 g2(grid, (unsigned)cdiv(dim, sw));
  const int g4 = (sw / 4 + WAVE - 1) / WAVE;
#define SEG_LAUNCH(G)                                                                             \
  do {                                                                                            \
    seg_tile_kernel<T, DyT, MODE, G><<<g2, 256, 0, s>>>(ki, vi, dy, n, dim, sw, rows, w.partial,  \
                                                        fin);                                     \
    seg_tile_finish_kernel<T, MODE, G><<<g2, 256, 0, s>>>(ki, n, dim, sw, rows, w.partial, fin);  \
  } while (0)
  switch (g4) {
    case 1: SEG_LAUNCH(1); break;
    case 2: SEG_LAUNCH(2); break;
    case 3: SEG_LAUNCH(3); break;
    case 4: SEG_LAUNCH(4); break;
    case 5: case 6: SEG_LAUNCH(6); break;
    case 7: case 8: SEG_LAUNCH(8); break;
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
