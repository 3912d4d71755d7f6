// The step entry points: parameter layout, workspace planning, context creation and the
// forward + hand-written backward of the decoder ("$1000 tier nanochat run" discussion,
// GPT.forward of the posted model; backward is the chain rule of each op).
#include <stdio.h>
#include <string.h>

#include <string>
#include <algorithm>
#include <type_traits>
#include <vector>

#include "gemm.h"

namespace gpt {

Layout make_layout(const gpt_config& c) {
  Layout L;
  long long off = 0;
  auto add = [&](const std::string& n, long long r, long long k) {
    L.e.push_back({n, off, r, k});
    long long at = off;
    off = align_elems(off + r * k);
    return at;
  };
  const long long D = c.d_model, F = c.d_mlp, V = c.vocab;
  L.wte = add("wte", V, D);
  for (int l = 0; l < c.n_layer; ++l) {
    std::string p = "h" + std::to_string(l) + ".";
    L.wqkv.push_back(add(p + "wqkv", 3 * D, D));
    L.wo.push_back(add(p + "wo", D, D));
    L.wfc.push_back(add(p + "wfc", F, D));
    L.wpr.push_back(add(p + "wpr", D, F));
  }
  L.lm_head = add("lm_head", V, D);
  if (c.has_trigram) L.wtri = add("wtri", D, D);
  L.total = off;
  return L;
}

gpt_status validate(const gpt_config* c) {
  if (!c) return fail(GPT_EINVAL, "config is null");
  if (c->n_layer < 1 || c->d_model < 1 || c->n_head < 1 || c->head_dim < 1 || c->d_mlp < 1 ||
      c->vocab < 1 || c->seq_len < 1 || c->batch < 1)
    return fail(GPT_ESHAPE, "every size in the config must be positive");
  if (c->n_kv_head != c->n_head) return fail(GPT_ESHAPE, "n_kv_head must equal n_head");
  if (c->n_head * c->head_dim != c->d_model) return fail(GPT_ESHAPE, "d_model != n_head * head_dim");
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(GPT_ESHAPE, "head_dim must be 32, 64 or 128");
  if (c->d_model % 64 || c->d_mlp % 64 || c->vocab % 64)
    return fail(GPT_ESHAPE, "d_model, d_mlp and vocab must be multiples of 64");
  if (c->d_model > 2048) return fail(GPT_ESHAPE, "d_model above 2048 is not supported");
  if (c->vocab > 65536) return fail(GPT_ESHAPE, "vocab above 65536 is not supported");
  if (c->seq_len % 64) return fail(GPT_ESHAPE, "seq_len must be a multiple of 64");
  if ((long long)c->batch * c->seq_len >= (1LL << 31) / 8)
    return fail(GPT_ESHAPE, "too many tokens per step");
  if (c->dtype != GPT_F32 && c->dtype != GPT_BF16) return fail(GPT_EINVAL, "bad dtype");
  if (c->ce_chunk_tokens < 0 || c->ce_chunk_tokens % 64)
    return fail(GPT_ESHAPE, "ce_chunk_tokens must be 0 or a positive multiple of 64");
  if (c->wgrad_stream < -1 || c->wgrad_stream > 1) return fail(GPT_EINVAL, "wgrad_stream must be -1, 0 or 1");
  if (!(c->rms_eps >= 0.f) || !(c->rope_base > 0.f) || !(c->softcap >= 0.f))
    return fail(GPT_ERANGE, "rms_eps, rope_base or softcap out of range");
  return GPT_OK;
}

namespace {

// Whether the blocks' weight gradients get a stream of their own (bf16 path only): the caller's
// choice, else where the MLP-up weight gradient's plan uses 128 x 128 tiles (two workgroups per
// CU, so the products of both streams share the CUs).  Measured on MI355X: GPT-2-small step
// 11.46 -> 10.61 ms; d32 (256 x 256 tiles, which fill the CUs, so only the ends of the launches
// overlap) 186.9 -> 186.3 ms, not worth stretching its kernels' individual durations.
bool use_wgrad_stream(const gpt_config& c) {
  if (c.dtype != GPT_BF16 || c.wgrad_stream < 0) return false;
  if (c.wgrad_stream > 0) return true;
  const long long n = (long long)c.batch * c.seq_len;
  return !gemm_detail::split_plan(c.d_mlp, c.d_model, (int)n).big;
}

// Tokens of one head/cross-entropy chunk: the caller's choice, capped so that the bf16/fp32
// logits chunk spans at most 2 GiB (the most one GEMM operand may span); by default all tokens
// when they fit.
long long ce_chunk_rows(const gpt_config& c) {
  const long long N = (long long)c.batch * c.seq_len;
  const long long esz = c.dtype == GPT_BF16 ? 2 : 4;
  long long rows = (2LL << 30) / ((long long)c.vocab * esz);
  rows = std::max<long long>(64, rows / 64 * 64);
  if (c.ce_chunk_tokens > 0) rows = std::min<long long>(rows, c.ce_chunk_tokens);
  return std::min(N, rows);
}

struct LayerBufs {
  float *x_in, *rstd_a, *rstd_qk, *lse, *x_mid, *rstd_b;
  void *a, *qkv, *o, *b, *act;
};

// Every device buffer of a step, carved from one workspace.  Element type sizes follow the
// dtype (T = bf16 or fp32); residual stream, statistics and gradients are fp32.
struct Plan {
  std::vector<LayerBufs> L;
  float *x_final, *rstd_f, *e_rstd, *dx, *db, *dqsum, *dU, *u, *de, *df, *loss_rows;
  void *f, *cos_t, *sin_t, *dx_t, *dact, *dO, *dqkv, *du_t, *logits;
  int32_t* tok_c;
  int *n_valid, *err;
  void* seg_ws;
  size_t seg_bytes;
  float* splitk;             // split-K partials of the weight-gradient GEMMs
  long long splitk_floats;
  long long ce_rows;
  long long* guard_tab;      // device copy of the guard offsets (first region, unguarded)
  std::vector<long long> guard_offs;
};

// Guards: one per region, at most this many for a config (per layer 11 regions, ~30 more).
long long guard_capacity(const gpt_config& c) { return 64 + 16LL * c.n_layer; }

Plan carve_plan(const gpt_config& c, Carver& cv) {
  Plan p;
  const long long N = (long long)c.batch * c.seq_len, D = c.d_model, F = c.d_mlp, H = c.n_head;
  // the guard table comes first; every region after it is followed by a guard, so a kernel
  // that writes past the end of its buffer overwrites a guard word (gpt_check_errors, bit 4)
  p.guard_tab = cv.take<long long>(guard_capacity(c));
  cv.guard = true;
  const size_t es = c.dtype == GPT_BF16 ? 2 : 4;
  auto T = [&](long long n) { return (void*)cv.take<char>(n * es); };
  const bool vadd = c.has_v_add || c.has_trigram;
  p.L.resize(c.n_layer);
  for (auto& l : p.L) {
    l.x_in = cv.take<float>(N * D);
    l.rstd_a = cv.take<float>(N);
    l.a = T(N * D);
    l.qkv = T(N * 3 * D);
    l.rstd_qk = cv.take<float>(N * 2 * H);
    l.o = T(N * D);
    l.lse = cv.take<float>(N * H);
    l.x_mid = cv.take<float>(N * D);
    l.rstd_b = cv.take<float>(N);
    l.b = T(N * D);
    l.act = T(N * F);
  }
  p.x_final = cv.take<float>(N * D);
  p.rstd_f = cv.take<float>(N);
  p.f = T(N * D);
  p.cos_t = T((long long)c.seq_len * c.head_dim / 2);
  p.sin_t = T((long long)c.seq_len * c.head_dim / 2);
  p.e_rstd = cv.take<float>(N);
  p.tok_c = cv.take<int32_t>(N);
  p.dx = cv.take<float>(N * D);
  p.dx_t = T(N * D);
  p.dact = T(N * F);
  p.db = cv.take<float>(N * D);
  p.dO = T(N * D);
  p.dqkv = T(N * 3 * D);
  p.dqsum = cv.take<float>(N * H);
  p.u = vadd ? cv.take<float>(N * D) : nullptr;
  p.dU = vadd ? cv.take<float>(N * D) : nullptr;
  p.du_t = c.has_trigram ? T(N * D) : nullptr;
  p.de = cv.take<float>(N * D);
  p.ce_rows = ce_chunk_rows(c);
  p.logits = T(p.ce_rows * c.vocab);
  p.df = cv.take<float>(N * D);
  p.loss_rows = cv.take<float>(N);
  p.n_valid = cv.take<int>(64);
  p.err = p.n_valid ? p.n_valid + 16 : nullptr;  // sizing carves hand out null pointers
  p.seg_bytes = segsum_workspace_bytes(N, (int)D);
  p.seg_ws = cv.take<char>(p.seg_bytes);
  p.splitk_floats = 0;
  if (c.dtype == GPT_BF16) {
    const int n = (int)N, d = (int)D, f = (int)F;
    const long long need[] = {gemm_wgrad_ws_floats(3 * d, d, n), gemm_wgrad_ws_floats(d, d, n),
                              gemm_wgrad_ws_floats(d, f, n), gemm_wgrad_ws_floats(f, d, n),
                              gemm_wgrad_ws_floats(c.vocab, d, (int)p.ce_rows),
                              // the LM head's input gradient (fp32 output, K = vocab)
                              gemm_wgrad_ws_floats((int)p.ce_rows, d, c.vocab)};
    for (long long x : need) p.splitk_floats = std::max(p.splitk_floats, x);
  }
  p.splitk = p.splitk_floats ? cv.take<float>(p.splitk_floats) : nullptr;
  p.guard_offs.assign(cv.guards.begin(), cv.guards.end());
  return p;
}

}  // namespace
}  // namespace gpt

struct gpt_ctx {
  gpt_config cfg;
  gpt::Layout layout;
  gpt::Plan plan;
  void* ws;
  size_t ws_bytes;
  gpt::Prof prof;
  // Weight gradients of the blocks on a stream of their own (when `side` is set), so that they
  // run beside the input-gradient chain; fork: the side stream waits for the caller's stream so
  // far; ev_dw / ev_ow: the caller's stream waits for the down / out weight gradient of a layer
  // before overwriting the gradient rows they read; ev_end: the join after the last layer.
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, ev_dw = nullptr, ev_ow = nullptr, ev_end = nullptr;
  ~gpt_ctx() {
    for (hipEvent_t e : {fork, ev_dw, ev_ow, ev_end})
      if (e) (void)hipEventDestroy(e);
    if (side) (void)hipStreamDestroy(side);
  }
};

namespace gpt {
namespace {

template <typename T>
gpt_status run_step(gpt_ctx* ctx, const int32_t* tokens, const int32_t* targets, const T* P,
                    float* G, float grad_scale, int accumulate, const T* x0_add, const T* v_add,
                    const T* tri_rows, T* d_x0_add, T* d_v_add, float* loss, hipStream_t s) {
  const gpt_config& c = ctx->cfg;
  const Layout& Ly = ctx->layout;
  Plan& p = ctx->plan;
  Prof& prof = ctx->prof;
  const long long N = (long long)c.batch * c.seq_len;
  const int D = c.d_model, F = c.d_mlp, V = c.vocab, H = c.n_head, hd = c.head_dim;
  const int Lc = c.n_layer, Tn = c.seq_len, Bn = c.batch;
  const int beta = accumulate ? 1 : 0;
  const bool vadd = c.has_v_add || c.has_trigram;
  const float eps = c.rms_eps;
  const double es = sizeof(T);
  const double ND = (double)N * D;
  const double pairs = (double)Bn * H * Tn * (Tn + 1) / 2.0;  // causal (query, key) pairs
  const T* cos_t = (const T*)p.cos_t;
  const T* sin_t = (const T*)p.sin_t;
  // Run one stage on stream `on`; with profiling on, bracket it by events and record its
  // algorithmic work.
  auto run_on = [&](hipStream_t on, const char* name, double flops, double bytes,
                    auto&& fn) -> gpt_status {
    if (!prof.on) return fn();
    hipEvent_t e0 = prof.get(), e1 = prof.get();
    if (!e0 || !e1) return fail(GPT_EHIP, "profiling: hipEventCreate failed");
    (void)hipEventRecord(e0, on);
    gpt_status st = fn();
    (void)hipEventRecord(e1, on);
    prof.recs.push_back({name, flops, bytes, e0, e1});
    return st;
  };
  auto run = [&](const char* name, double flops, double bytes, auto&& fn) -> gpt_status {
    return run_on(s, name, flops, bytes, fn);
  };
  // The blocks' weight gradients go to ws (the side stream, or s itself): fork() makes ws wait
  // for everything issued to s so far; mark(e) records e after what ws holds so far, and
  // await_mark(e) makes s wait for it.  A profiled step stays on one stream, so that each
  // stage's events time its own kernels.
  const bool side = ctx->side != nullptr && !prof.on;
  hipStream_t ws = side ? ctx->side : s;
  // bf16: the q/k/v and out weight gradients as one paired launch when their 256 x 256 tiles
  // together make a whole round of the CUs (d32: 192 + 64 of 256); a function of the shape, so
  // the results do not depend on the streams
  bool pair_wgrads = false;
  if (std::is_same<T, bf16>::value) {
    const long long t_qkv = cdiv(3LL * D, 256) * cdiv((long long)D, 256);
    const long long t_out = cdiv((long long)D, 256) * cdiv((long long)D, 256);
    pair_wgrads = t_qkv % 8 == 0 && t_qkv + t_out == (long long)gemm_detail::resident_cus();
  }
  auto fork = [&]() -> gpt_status {
    if (!side) return GPT_OK;
    if (hipEventRecord(ctx->fork, s) != hipSuccess || hipStreamWaitEvent(ws, ctx->fork, 0) != hipSuccess)
      return fail(GPT_EHIP, "weight-gradient stream: fork failed");
    return GPT_OK;
  };
  auto mark = [&](hipEvent_t e) -> gpt_status {
    if (side && hipEventRecord(e, ws) != hipSuccess) return fail(GPT_EHIP, "weight-gradient stream: record failed");
    return GPT_OK;
  };
  auto await_mark = [&](hipEvent_t e) -> gpt_status {
    if (side && hipStreamWaitEvent(s, e, 0) != hipSuccess) return fail(GPT_EHIP, "weight-gradient stream: wait failed");
    return GPT_OK;
  };
  auto mm = [](double m, double n, double k) { return 2.0 * m * n * k; };
#define TRY(x)                          \
  do {                                  \
    gpt_status st_ = (x);               \
    if (st_ != GPT_OK) return st_;      \
  } while (0)
#define STAGE(name, flops, bytes, ...) TRY(run(name, flops, bytes, [&]() { return __VA_ARGS__; }))
#define SIDE_STAGE(name, flops, bytes, ...) \
  TRY(run_on(ws, name, flops, bytes, [&]() { return __VA_ARGS__; }))

  // value addend u = v_add + tri_rows wtri^T (fp32), shared by every layer
  const float* u = nullptr;
  if (c.has_trigram) {
    STAGE("tri_proj", mm(N, D, D), 0,
          gemm<G_TRI, T>(true, true, (int)N, D, D, tri_rows, D, P + Ly.wtri, D,
                         EpiAddRows<T>{c.has_v_add ? v_add : nullptr, p.u, D}, s));
    u = p.u;
  } else if (c.has_v_add) {
    STAGE("vadd_cast", 0, ND * (es + 4), launch_accum_rows<T>(p.u, v_add, D, N, D, 0, s));
    u = p.u;
  }
  STAGE("count_targets", 0, 4.0 * N, launch_count_targets(targets, N, V, p.n_valid, p.err, s));
  STAGE("embed_fwd", 0, ND * (es + (c.has_x0_add ? es : 0) + 4) + 12.0 * N,
        launch_embed_fwd<T>(tokens, P + Ly.wte, c.has_x0_add ? x0_add : nullptr, p.L[0].x_in,
                            p.e_rstd, p.tok_c, p.err, N, D, V, eps, s));

  // The bf16 path applies rotary + QK-norm in the QKV projection's epilogue when every wave
  // tile of 128 projection columns lies inside one of the q, k, v blocks (d_model a multiple of
  // 128); otherwise (and on the fp32 path) the projection is stored and a separate kernel
  // rotates and normalizes q and k in place.  Both leave the same tensors for the backward.
  const bool fuse_rope = std::is_same<T, bf16>::value && D % 128 == 0;
  auto qkv_rope = [&](const T* w, const T* a, T* qkv, float* rstd_qk) -> gpt_status {
    if constexpr (std::is_same<T, bf16>::value) {
      auto go = [&](auto qkn_c, auto vadd_c) {
        constexpr bool QKN = decltype(qkn_c)::value, VADD = decltype(vadd_c)::value;
        const EpiQKVRope<T, QKN, VADD> e{qkv, 3LL * D, cos_t, sin_t, rstd_qk, u, D, D, hd, Tn,
                                         H, eps};
        return gemm<G_QKV, T>(true, true, (int)N, 3 * D, D, a, D, w, D, e, s);
      };
      if (c.qk_norm) return u ? go(std::true_type(), std::true_type()) : go(std::true_type(), std::false_type());
      return u ? go(std::false_type(), std::true_type()) : go(std::false_type(), std::false_type());
    } else {
      return fail(GPT_EINVAL, "fused rotary projection is bf16 only");
    }
  };

  // ---------------- forward
  for (int l = 0; l < Lc; ++l) {
    LayerBufs& b = p.L[l];
    T *a = (T*)b.a, *qkv = (T*)b.qkv, *o = (T*)b.o, *bb = (T*)b.b, *act = (T*)b.act;
    float* x_out = l + 1 < Lc ? p.L[l + 1].x_in : p.x_final;
    STAGE("rmsnorm_fwd", 0, ND * (4 + es) + 4.0 * N,
          launch_rms_fwd<T>(b.x_in, a, b.rstd_a, N, D, eps, s));
    if (fuse_rope) {
      // rotary + QK-norm in the projection's epilogue: one pass, q and k never stored unrotated
      STAGE("qkv_rope_fwd", mm(N, 3 * D, D), 0,
            qkv_rope(P + Ly.wqkv[l], a, qkv, b.rstd_qk));
    } else {
      STAGE("qkv_fwd", mm(N, 3 * D, D), 0,
            gemm<G_QKV, T>(true, true, (int)N, 3 * D, D, a, D, P + Ly.wqkv[l], D,
                           EpiQKV<T>{qkv, 3LL * D, u, D, 2 * D}, s));
      STAGE("rope_qknorm_fwd", 0, 4.0 * ND * es + 8.0 * N * H,
            launch_rope_qknorm_fwd<T>(qkv, cos_t, sin_t, b.rstd_qk, N, Tn, H, hd, c.qk_norm, eps, s));
    }
    STAGE("attn_fwd", 4.0 * pairs * hd, 0,
          launch_attn_fwd<T>(qkv, o, b.lse, Bn, Tn, H, hd, s, c.qk_norm));
    STAGE("out_fwd", mm(N, D, D), 0,
          gemm<G_OUT, T>(true, true, (int)N, D, D, o, D, P + Ly.wo[l], D,
                         EpiResid{b.x_in, b.x_mid, D}, s));
    STAGE("rmsnorm_fwd", 0, ND * (4 + es) + 4.0 * N,
          launch_rms_fwd<T>(b.x_mid, bb, b.rstd_b, N, D, eps, s));
    STAGE("up_fwd", mm(N, F, D), 0,
          gemm<G_UP, T>(true, true, (int)N, F, D, bb, D, P + Ly.wfc[l], D,
                        EpiRelu2<T>{act, F}, s));
    STAGE("down_fwd", mm(N, D, F), 0,
          gemm<G_DOWN, T>(true, true, (int)N, D, F, act, F, P + Ly.wpr[l], F,
                          EpiResid{b.x_mid, x_out, D}, s));
  }
  T* f = (T*)p.f;
  STAGE("rmsnorm_fwd", 0, ND * (4 + es) + 4.0 * N,
        launch_rms_fwd<T>(p.x_final, f, p.rstd_f, N, D, eps, s));

  // ---------------- LM head + softcapped cross-entropy, chunked over tokens
  T* z = (T*)p.logits;
  const T* wh = P + Ly.lm_head;
  for (long long c0 = 0; c0 < N; c0 += p.ce_rows) {
    const int rows = (int)std::min<long long>(p.ce_rows, N - c0);
    STAGE("head_fwd", mm(rows, V, D), 0,
          gemm<G_HEAD, T>(true, true, rows, V, D, f + c0 * D, D, wh, D, EpiStore<T>{z, V}, s));
    STAGE("softcap_ce", 0, 2.0 * rows * V * es + 8.0 * rows,
          launch_ce<T>(z, V, targets + c0, rows, V, c.softcap, grad_scale, p.n_valid,
                       p.loss_rows + c0, s));
    STAGE("head_dgrad", mm(rows, D, V), 0,
          gemm_wgrad<G_HEAD_DGRAD, T>(true, false, rows, D, V, z, V, wh, D,
                                      EpiStoreF32{p.df + c0 * D, D, 0}, p.splitk,
                                      p.splitk_floats, s));
    STAGE("head_wgrad", mm(V, D, rows), 0,
          gemm_wgrad<G_HEAD_WGRAD, T>(false, false, V, D, rows, z, V, f + c0 * D, D,
                                      EpiStoreF32{G + Ly.lm_head, D, (beta || c0 > 0) ? 1 : 0},
                                      p.splitk, p.splitk_floats, s));
  }
  STAGE("loss_reduce", 0, 4.0 * N, launch_loss_reduce(p.loss_rows, N, p.n_valid, loss, s));
  T* dx_t = (T*)p.dx_t;
  STAGE("rmsnorm_bwd", 0, ND * (12 + es) + 4.0 * N,
        launch_rms_bwd<T>(p.x_final, p.rstd_f, p.df, nullptr, p.dx, dx_t, N, D, s));

  // ---------------- backward through the blocks
  T *dact = (T*)p.dact, *dO = (T*)p.dO, *dqkv = (T*)p.dqkv;
  for (int l = Lc - 1; l >= 0; --l) {
    LayerBufs& b = p.L[l];
    const T *a = (const T*)b.a, *qkv = (const T*)b.qkv, *o = (const T*)b.o, *bb = (const T*)b.b,
            *act = (const T*)b.act;
    // MLP: x_out = x_mid + relu(b Wfc^T)^2 Wpr^T.  With the side stream, the weight gradients
    // of a layer run beside its input-gradient chain; s waits for the down (out) weight gradient
    // before the norm backward overwrites the dx_t rows it reads.  The other buffers a weight
    // gradient reads (dact, dqkv) are next written one layer later, after s has already waited
    // for a later item of the in-order side stream.
    TRY(fork());
    SIDE_STAGE("down_wgrad", mm(D, F, N), 0,
               gemm_wgrad<G_DOWN_WGRAD, T>(false, false, D, F, (int)N, dx_t, D, act, F,
                                           EpiStoreF32{G + Ly.wpr[l], F, beta}, p.splitk,
                                           p.splitk_floats, ws));
    TRY(mark(ctx->ev_dw));
    STAGE("down_dgrad", mm(N, F, D), 0,
          gemm<G_DOWN_DGRAD, T>(true, false, (int)N, F, D, dx_t, D, P + Ly.wpr[l], F,
                                EpiDRelu2<T>{act, dact, F}, s));
    TRY(fork());
    SIDE_STAGE("up_wgrad", mm(F, D, N), 0,
               gemm_wgrad<G_UP_WGRAD, T>(false, false, F, D, (int)N, dact, F, bb, D,
                                         EpiStoreF32{G + Ly.wfc[l], D, beta}, p.splitk,
                                         p.splitk_floats, ws));
    STAGE("up_dgrad", mm(N, D, F), 0,
          gemm<G_UP_DGRAD, T>(true, false, (int)N, D, F, dact, F, P + Ly.wfc[l], D,
                              EpiStoreF32{p.db, D, 0}, s));
    TRY(await_mark(ctx->ev_dw));
    STAGE("rmsnorm_bwd", 0, ND * (16 + es) + 4.0 * N,
          launch_rms_bwd<T>(b.x_mid, b.rstd_b, p.db, p.dx, p.dx, dx_t, N, D, s));
    // attention: x_mid = x_in + O Wo^T
    if (!pair_wgrads) {
      TRY(fork());
      SIDE_STAGE("out_wgrad", mm(D, D, N), 0,
                 gemm_wgrad<G_OUT_WGRAD, T>(false, false, D, D, (int)N, dx_t, D, o, D,
                                            EpiStoreF32{G + Ly.wo[l], D, beta}, p.splitk,
                                            p.splitk_floats, ws));
      TRY(mark(ctx->ev_ow));
    }
    STAGE("out_dgrad", mm(N, D, D), 0,
          gemm<G_OUT_DGRAD, T>(true, false, (int)N, D, D, dx_t, D, P + Ly.wo[l], D,
                               EpiStore<T>{dO, D}, s));
    STAGE("attn_bwd_dq", 2.0 * pairs * hd, 0,
          launch_attn_bwd_stage<T>(0, qkv, o, dO, b.lse, p.dqsum, dqkv, Bn, Tn, H, hd, s));
    STAGE("attn_bwd_dkdv", 8.0 * pairs * hd, 0,
          launch_attn_bwd_stage<T>(1, qkv, o, dO, b.lse, p.dqsum, dqkv, Bn, Tn, H, hd, s));
    STAGE("rope_qknorm_bwd", 0, 6.0 * ND * es + 8.0 * N * H,
          launch_rope_qknorm_bwd<T>(dqkv, qkv, cos_t, sin_t, b.rstd_qk, N, Tn, H, hd, c.qk_norm, s));
    if (vadd)
      STAGE("dvadd_accum", 0, ND * (es + (l != Lc - 1 ? 8 : 4)),
            launch_accum_rows<T>(p.dU, dqkv + 2 * D, 3LL * D, N, D, l != Lc - 1, s));
    if (pair_wgrads) {
      // the out weight gradient, deferred to here, runs in one launch with the q/k/v one:
      // together their 256 x 256 tiles fill one round of the CUs (dx_t, which the out product
      // reads, is rewritten only by the norm backward below)
      TRY(fork());
      if constexpr (std::is_same<T, bf16>::value)
        SIDE_STAGE("qkv_out_wgrad", mm(3 * D, D, N) + mm(D, D, N), 0,
                   gemm_wgrad_pair<G_QKV_OUT_WGRAD>(3 * D, D, (int)N, dqkv, 3 * D, a, D,
                                                    EpiStoreF32{G + Ly.wqkv[l], D, beta}, D, D,
                                                    (int)N, dx_t, D, o, D,
                                                    EpiStoreF32{G + Ly.wo[l], D, beta}, ws));
      TRY(mark(ctx->ev_ow));
    } else {
      TRY(fork());
      SIDE_STAGE("qkv_wgrad", mm(3 * D, D, N), 0,
                 gemm_wgrad<G_QKV_WGRAD, T>(false, false, 3 * D, D, (int)N, dqkv, 3 * D, a, D,
                                            EpiStoreF32{G + Ly.wqkv[l], D, beta}, p.splitk,
                                            p.splitk_floats, ws));
    }
    STAGE("qkv_dgrad", mm(N, D, 3 * D), 0,
          gemm<G_QKV_DGRAD, T>(true, false, (int)N, D, 3 * D, dqkv, 3 * D, P + Ly.wqkv[l], D,
                               EpiStoreF32{p.db, D, 0}, s));
    TRY(await_mark(ctx->ev_ow));
    STAGE("rmsnorm_bwd", 0, ND * (16 + es) + 4.0 * N,
          launch_rms_bwd<T>(b.x_in, b.rstd_a, p.db, p.dx, p.dx, dx_t, N, D, s));
  }
  // every weight gradient of the blocks is written (and the split-K workspace free) from here on
  TRY(mark(ctx->ev_end));
  TRY(await_mark(ctx->ev_end));

  // ---------------- embedding, x0 addend, value addend
  if (c.has_x0_add && d_x0_add)
    STAGE("cast", 0, ND * (4 + es), launch_cast<T>(d_x0_add, p.dx, N * D, s));
  STAGE("embed_bwd", 0, ND * (es + 8) + 8.0 * N,
        launch_embed_bwd<T>(p.tok_c, P + Ly.wte, p.e_rstd, p.dx, p.de, N, D, s));
  if (!accumulate)
    STAGE("fill", 0, 4.0 * V * D, launch_fill(G + Ly.wte, (long long)V * D, 0.f, s));
  STAGE("wte_segsum", 0, ND * 4 * 2,
        segsum_grad(p.tok_c, p.de, N, D, G + Ly.wte, V, 1, p.seg_ws, p.seg_bytes, s));
  if (vadd) {
    if (c.has_v_add && d_v_add)
      STAGE("cast", 0, ND * (4 + es), launch_cast<T>(d_v_add, p.dU, N * D, s));
    if (c.has_trigram) {
      T* du_t = (T*)p.du_t;
      STAGE("cast", 0, ND * (4 + es), launch_cast<T>(du_t, p.dU, N * D, s));
      STAGE("tri_wgrad", mm(D, D, N), 0,
            gemm_wgrad<G_TRI_WGRAD, T>(false, false, D, D, (int)N, du_t, D, tri_rows, D,
                                       EpiStoreF32{G + Ly.wtri, D, beta}, p.splitk,
                                       p.splitk_floats, s));
    }
  }
#undef SIDE_STAGE
#undef STAGE
#undef TRY
  return GPT_OK;
}

}  // namespace
}  // namespace gpt

using namespace gpt;

extern "C" {

gpt_status gpt_param_layout(const gpt_config* cfg, gpt_tensor_desc* out, int32_t* count,
                            int64_t* total_elems) {
  gpt_status st = validate(cfg);
  if (st != GPT_OK) return st;
  if (!count) return fail(GPT_EINVAL, "gpt_param_layout: count is null");
  Layout L = make_layout(*cfg);
  if (total_elems) *total_elems = L.total;
  if (!out) {
    *count = (int32_t)L.e.size();
    return GPT_OK;
  }
  if (*count < (int32_t)L.e.size()) return fail(GPT_EINVAL, "gpt_param_layout: out too small");
  for (size_t i = 0; i < L.e.size(); ++i) {
    memset(&out[i], 0, sizeof(out[i]));
    snprintf(out[i].name, sizeof(out[i].name), "%s", L.e[i].name.c_str());
    out[i].offset_elems = L.e[i].off;
    out[i].ndim = 2;
    out[i].shape[0] = L.e[i].rows;
    out[i].shape[1] = L.e[i].cols;
  }
  *count = (int32_t)L.e.size();
  return GPT_OK;
}

gpt_status gpt_workspace_bytes(const gpt_config* cfg, size_t* bytes) {
  gpt_status st = validate(cfg);
  if (st != GPT_OK) return st;
  if (!bytes) return fail(GPT_EINVAL, "gpt_workspace_bytes: bytes is null");
  Carver cv(nullptr, 0);
  carve_plan(*cfg, cv);
  *bytes = cv.size();
  return GPT_OK;
}

gpt_status gpt_init(const gpt_config* cfg, void* workspace, size_t ws_bytes, hipStream_t stream,
                    gpt_ctx** out) {
  gpt_status st = validate(cfg);
  if (st != GPT_OK) return st;
  if (!out) return fail(GPT_EINVAL, "gpt_init: out is null");
  if (!workspace) return fail(GPT_EWORKSPACE, "gpt_init: workspace is null");
  if (((uintptr_t)workspace) % 256) return fail(GPT_EINVAL, "gpt_init: workspace not 256-byte aligned");
  if (cfg->dtype == GPT_F32 && cfg->head_dim > 64)
    return fail(GPT_ESHAPE, "gpt_init: the fp32 path supports head_dim 32 or 64");
  Carver cv(workspace, ws_bytes);
  Plan plan = carve_plan(*cfg, cv);
  if (!cv.ok) return fail(GPT_EWORKSPACE, "gpt_init: workspace smaller than gpt_workspace_bytes");
  gpt_ctx* ctx = new gpt_ctx{*cfg, make_layout(*cfg), plan, workspace, ws_bytes};
  if (use_wgrad_stream(*cfg)) {
    bool ok = hipStreamCreateWithFlags(&ctx->side, hipStreamNonBlocking) == hipSuccess;
    for (hipEvent_t* e : {&ctx->fork, &ctx->ev_dw, &ctx->ev_ow, &ctx->ev_end})
      ok = ok && hipEventCreateWithFlags(e, hipEventDisableTiming) == hipSuccess;
    if (!ok) {
      delete ctx;
      return fail(GPT_EHIP, "gpt_init: weight-gradient stream or events could not be created");
    }
  }
  if (cfg->dtype == GPT_BF16)
    st = launch_rope_table<bf16>((bf16*)plan.cos_t, (bf16*)plan.sin_t, cfg->seq_len, cfg->head_dim,
                                 cfg->rope_base, stream);
  else
    st = launch_rope_table<float>((float*)plan.cos_t, (float*)plan.sin_t, cfg->seq_len,
                                  cfg->head_dim, cfg->rope_base, stream);
  if (st == GPT_OK) st = launch_fill((float*)plan.n_valid, 64, 0.f, stream);
  if (st == GPT_OK) {
    // the guard table (the context keeps the host copy alive for the asynchronous copy)
    const int ng = (int)ctx->plan.guard_offs.size();
    if (ng > guard_capacity(*cfg)) st = fail(GPT_ESHAPE, "gpt_init: too many workspace regions");
    else if (hipMemcpyAsync(ctx->plan.guard_tab, ctx->plan.guard_offs.data(), ng * sizeof(long long),
                            hipMemcpyHostToDevice, stream) != hipSuccess)
      st = fail(GPT_EHIP, "gpt_init: guard table copy failed");
    else st = launch_guards((char*)workspace, ctx->plan.guard_tab, ng, nullptr, 0, stream);
  }
  if (st != GPT_OK) {
    delete ctx;
    return st;
  }
  *out = ctx;
  return GPT_OK;
}

gpt_status gpt_fwd_bwd(gpt_ctx* ctx, const int32_t* tokens, const int32_t* targets,
                       const void* params, float* grads, float grad_scale, int32_t accumulate,
                       const void* x0_add, const void* v_add, const void* tri_rows,
                       void* d_x0_add, void* d_v_add, float* loss, hipStream_t stream) {
  if (!ctx) return fail(GPT_EINVAL, "gpt_fwd_bwd: ctx is null");
  if (!tokens || !targets || !params || !grads || !loss)
    return fail(GPT_EINVAL, "gpt_fwd_bwd: null tokens, targets, params, grads or loss");
  const gpt_config& c = ctx->cfg;
  if (c.has_x0_add && !x0_add) return fail(GPT_EINVAL, "gpt_fwd_bwd: x0_add required");
  if (c.has_v_add && !v_add) return fail(GPT_EINVAL, "gpt_fwd_bwd: v_add required");
  if (c.has_trigram && !tri_rows) return fail(GPT_EINVAL, "gpt_fwd_bwd: tri_rows required");
  if (accumulate != 0 && accumulate != 1) return fail(GPT_EINVAL, "gpt_fwd_bwd: accumulate must be 0 or 1");
  const uintptr_t al = (uintptr_t)params | (uintptr_t)grads | (uintptr_t)x0_add | (uintptr_t)v_add |
                       (uintptr_t)tri_rows | (uintptr_t)d_x0_add | (uintptr_t)d_v_add;
  if (al % 16) return fail(GPT_EINVAL, "gpt_fwd_bwd: buffers must be 16-byte aligned");
  if (c.dtype == GPT_BF16)
    return run_step<bf16>(ctx, tokens, targets, (const bf16*)params, grads, grad_scale, accumulate,
                          (const bf16*)x0_add, (const bf16*)v_add, (const bf16*)tri_rows,
                          (bf16*)d_x0_add, (bf16*)d_v_add, loss, stream);
  return run_step<float>(ctx, tokens, targets, (const float*)params, grads, grad_scale, accumulate,
                         (const float*)x0_add, (const float*)v_add, (const float*)tri_rows,
                         (float*)d_x0_add, (float*)d_v_add, loss, stream);
}

gpt_status gpt_check_errors(gpt_ctx* ctx, hipStream_t stream, int32_t* flags) {
  if (!ctx || !flags) return fail(GPT_EINVAL, "gpt_check_errors: null argument");
  gpt_status gs = launch_guards((char*)ctx->ws, ctx->plan.guard_tab,
                                (int)ctx->plan.guard_offs.size(), ctx->plan.err, 1, stream);
  if (gs != GPT_OK) return gs;
  int32_t h = 0;
  if (hipMemcpyAsync(&h, ctx->plan.err, sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return fail(GPT_EHIP, "gpt_check_errors: copy failed");
  *flags = h;
  gpt_status st = launch_fill((float*)ctx->plan.err, 1, 0.f, stream);
  return st;
}

gpt_status gpt_profile(gpt_ctx* ctx, int32_t enable) {
  if (!ctx) return fail(GPT_EINVAL, "gpt_profile: ctx is null");
  ctx->prof.on = enable != 0;
  return GPT_OK;
}

gpt_status gpt_profile_read(gpt_ctx* ctx, gpt_profile_entry* out, int32_t* count) {
  if (!ctx || !count) return fail(GPT_EINVAL, "gpt_profile_read: null argument");
  return prof_read(ctx->prof, out, count, "gpt_profile_read");
}

gpt_status gpt_destroy(gpt_ctx* ctx) {
  delete ctx;
  return GPT_OK;
}

}  // extern "C"
