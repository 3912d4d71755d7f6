/*
 * gpt.h -- C ABI of libgpt.so: one training step (forward + hand-written backward) of a
 * GPT-style decoder, and the hashed n-gram tables with their inlined sparse optimizer, on
 * AMD Instinct MI355X (gfx950).
 *
 * What is computed (definitions from the pages; each entry point cites its own):
 *   - the decoder of the "$1000 tier nanochat run" discussion (nanochat #8, the GPT class a
 *     commenter posted): x = norm(wte[idx]); per block x += attn(norm(x)), x += mlp(norm(x));
 *     norm(x); untied lm_head; logits softcap 15*tanh(z/15); mean cross-entropy over targets
 *     != -1.  norm is RMSNorm without weight (modded-nanogpt README: "Removed all affine scale
 *     and bias parameters"), attention has half-split rotary embeddings, QK-norm and a causal
 *     mask, the MLP activation is ReLU^2 (README: "ReLU^2 activation").
 *   - the decoder-rtx tables (Chris McCormick posts, baseline-4 thread): a hashed bigram row
 *     added to x0, a hashed bigram row and a projected frozen trigram row added to the
 *     attention values, and a sparse optimizer "with no first moment and only per-row
 *     magnitude" applied inside backward so that no table-gradient buffer exists.
 *
 * Conventions (all entry points):
 *   - Pointers are DEVICE pointers unless marked [host].  All memory is caller-owned; the
 *     library never allocates device memory and never synchronises the stream, except where a
 *     function says so.  Every launch is ordered on the stream argument.
 *   - Row-major everywhere.  Activations are token-major [N, .] with N = batch * seq_len,
 *     token (b, t) at row b * seq_len + t.  Weights are [out, in] (nn.Linear layout).
 *   - Arguments are validated before any launch; a failing call returns a negative status
 *     and launches nothing.  Launch failures return GPT_EHIP.  gpt_last_error() [host] gives
 *     a human-readable message for the last failure on the calling thread.
 *   - bf16 means IEEE bfloat16 storage; all bf16 stores round to nearest even from fp32.
 */
#ifndef GPT_H_
#define GPT_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPT_OK = 0,
  GPT_EINVAL = -1,      /* null pointer, bad enum, unsupported option */
  GPT_ESHAPE = -2,      /* a size or alignment the kernels do not support */
  GPT_ERANGE = -3,      /* a value out of range (detected on the host) */
  GPT_EWORKSPACE = -4,  /* workspace missing or smaller than the query said */
  GPT_EHIP = -5         /* a HIP launch or runtime call failed */
} gpt_status;

typedef enum { GPT_F32 = 0, GPT_BF16 = 1 } gpt_dtype;

/* Model configuration.  d_model = n_head * head_dim; n_kv_head must equal n_head (every
 * configuration on the pages uses as many key/value heads as query heads).
 * Supported: head_dim in {32, 64, 128}; d_model, d_mlp and vocab multiples of 64;
 * seq_len a multiple of 64; dtype GPT_BF16 (bf16 storage, fp32 accumulation, fp32 residual
 * stream and gradients) or GPT_F32 (everything fp32). */
typedef struct {
  int32_t n_layer, d_model, n_head, n_kv_head, head_dim, d_mlp, vocab, seq_len, batch;
  int32_t dtype;       /* gpt_dtype of parameters, activations and table addends */
  float rms_eps;       /* RMSNorm epsilon inside the square root (1e-6) */
  float rope_base;     /* rotary base (10000) */
  float softcap;       /* logit softcap c = s*tanh(z/s); 0 disables (15) */
  int32_t qk_norm;     /* 1: RMSNorm q and k per head after the rotation */
  int32_t has_x0_add;  /* 1: a per-token addend is added to x0 (after the embedding norm) */
  int32_t has_v_add;   /* 1: a per-token addend is added to the values of every layer */
  int32_t has_trigram; /* 1: gathered trigram rows, projected by wtri [D,D], add to values */
  int32_t ce_chunk_tokens; /* tokens per LM-head / cross-entropy chunk: 0 = as many as keep the
                              logits chunk within 2 GiB (all tokens of every shipped workload);
                              otherwise a multiple of 64.  Smaller chunks shrink the workspace
                              (the logits chunk is [chunk, vocab] in dtype); the result does not
                              depend on the chunking beyond fp32 summation order of the head's
                              weight gradient. */
  int32_t wgrad_stream;    /* where the blocks' weight-gradient products run in the backward
                              (bf16 only; fp32 always uses the caller's stream): 1 = a stream of
                              their own, created by gpt_init, beside the input-gradient chain
                              (the caller's stream waits for it before gpt_fwd_bwd's work
                              returns to it); -1 = the caller's stream only; 0 = the library's
                              choice (its own stream where those products use 128 x 128 tiles,
                              as in the GPT-2-small shapes).  Profiled steps (gpt_profile) stay
                              on the caller's stream.  Results are bitwise the same either way:
                              only the overlap of independent kernels changes. */
} gpt_config;

/* One entry of the flat parameter layout. */
typedef struct {
  char name[48];        /* "wte", "h<l>.wqkv", "h<l>.wo", "h<l>.wfc", "h<l>.wpr", "lm_head", "wtri" */
  int64_t offset_elems; /* offset in elements into the flat buffer (a multiple of 64) */
  int32_t ndim;         /* always 2 */
  int64_t shape[2];     /* [rows, cols]; h<l>.wqkv stacks the q, k and v projections [3D, D] */
} gpt_tensor_desc;

typedef struct gpt_ctx gpt_ctx;

/* Flat parameter layout of `cfg` [host, no GPU work].  Order: wte [V,D]; per layer l:
 * h<l>.wqkv [3D,D], h<l>.wo [D,D], h<l>.wfc [F,D], h<l>.wpr [D,F]; lm_head [V,D]; wtri [D,D]
 * if has_trigram.  `out` may be NULL to query the count; otherwise it must hold *count
 * entries on entry ([host] in/out: capacity in, number written out).  `total_elems` [host,
 * optional] receives the flat buffer length.  The gradient buffer uses the same layout. */
gpt_status gpt_param_layout(const gpt_config* cfg, gpt_tensor_desc* out, int32_t* count,
                            int64_t* total_elems);

/* Device workspace, in bytes, that gpt_init needs for `cfg` [host].  It holds the activation
 * stash of every layer, the logits of the LM head, rotary tables and sort scratch. */
gpt_status gpt_workspace_bytes(const gpt_config* cfg, size_t* bytes);

/* Create a step context over a caller-provided workspace (256-byte aligned, at least
 * gpt_workspace_bytes).  Enqueues one kernel on `stream` that fills the rotary tables
 * (cos/sin of t * base^(-2i/head_dim), stored in `dtype`, as _precompute_rotary_embeddings
 * on the nanochat page).  When the weight gradients get a stream of their own (see
 * gpt_config.wgrad_stream) it also creates that stream (default priority) and four events,
 * released by gpt_destroy.  *out [host] receives the context.  Not thread-safe per context. */
gpt_status gpt_init(const gpt_config* cfg, void* workspace, size_t ws_bytes, hipStream_t stream,
                    gpt_ctx** out);

/* One forward + backward pass (GPT.forward on the nanochat page, then the chain rule).
 *   tokens   int32 [B,T]: input ids; targets int32 [B,T]: next-token ids, -1 = ignored.
 *            Ids outside [0, vocab) are clamped for addressing and reported by
 *            gpt_check_errors (they never fault).
 *   params   flat buffer in `dtype` per gpt_param_layout (read only).
 *   grads    flat fp32 buffer, same layout: the gradient of grad_scale * loss.  accumulate = 0
 *            overwrites every entry; accumulate = 1 adds to it (gradient accumulation).
 *   x0_add, v_add, tri_rows  [N,D] in `dtype`: gathered table rows (bigram_fwd with y = 0),
 *            required iff has_x0_add / has_v_add / has_trigram, else ignored.
 *            The value addend is u = v_add + tri_rows * wtri^T, added to v in every layer.
 *   d_x0_add, d_v_add  [N,D] in `dtype` (may be NULL): per-token gradients of
 *            grad_scale * loss w.r.t. x0_add and v_add (u), always overwritten.  These feed
 *            bigram_bwd_update; no [rows, D] table gradient exists anywhere.
 *   loss     fp32 device scalar: mean cross-entropy over valid targets (not scaled).
 * Stream-ordered; never synchronises.  With the context's weight-gradient stream, that stream
 * first waits for `stream` and `stream` waits for it before the call's last launches, so
 * everything the call writes is ordered on `stream` as usual. */
gpt_status gpt_fwd_bwd(gpt_ctx* ctx, const int32_t* tokens, const int32_t* targets,
                       const void* params, float* grads, float grad_scale, int32_t accumulate,
                       const void* x0_add, const void* v_add, const void* tri_rows,
                       void* d_x0_add, void* d_v_add, float* loss, hipStream_t stream);

/* Bit flags of problems the kernels of this context detected since the last call:
 * 1 = an input token id outside [0, vocab); 2 = a target id outside [-1, vocab) (the offending
 * ids were clamped or ignored, so nothing faulted); 4 = a guard region of the workspace was
 * overwritten: every buffer gpt_init carves is followed by 256 guard bytes holding a known
 * pattern, checked here, so a kernel writing past the end of its buffer is reported.
 * Synchronises `stream`, then clears the flags.  flags [host]. */
gpt_status gpt_check_errors(gpt_ctx* ctx, hipStream_t stream, int32_t* flags);

/* Per-stage timing of gpt_fwd_bwd.  gpt_profile(ctx, 1) makes later steps bracket every launch
 * with two HIP events on the step's stream (a small overhead per launch); gpt_profile(ctx, 0)
 * stops recording.  gpt_profile_read synchronises on the recorded events, aggregates them by
 * stage name in order of first launch, clears them, and writes up to *count entries to `out`
 * [host] (*count [host] in: capacity, out: number of stages; out may be NULL to query).
 * flops and bytes are the stage's algorithmic work: 2*M*N*K per GEMM; causal attention
 * 4*pairs*hd forward, 8*pairs*hd for dK/dV and 2*pairs*hd for dQ (its recomputation of the
 * scores is not counted); and the bytes each memory-bound kernel must read and write once. */
typedef struct {
  char name[32];
  int32_t calls;
  float ms;
  double flops;
  double bytes;
} gpt_profile_entry;
gpt_status gpt_profile(gpt_ctx* ctx, int32_t enable);
gpt_status gpt_profile_read(gpt_ctx* ctx, gpt_profile_entry* out, int32_t* count);

gpt_status gpt_destroy(gpt_ctx* ctx);

/* ---- Dense optimizer step (the training script of the "$1000 tier nanochat run" discussion:
 * gradient clipping in its accumulation loop, setup_optimizers, the Muon class with
 * zeropower_via_newtonschulz5, get_lr_multiplier, get_muon_momentum; the modded-nanogpt README
 * for the bfloat16 Newton-Schulz iteration).  One call, after gpt_fwd_bwd has left the full
 * gradient in `grads`:
 *   1. norm = global L2 norm of grads; every gradient is scaled by f = min(1, grad_clip /
 *      (norm + 1e-6)) (f = 1 when grad_clip == 0).
 *   2. Adam (bias-corrected, decoupled weight decay) on wte with lr = lr_embedding * s * lr_mult
 *      and on lm_head with lr = lr_unembedding * s * lr_mult, s = (d_model / 768)^-1/2:
 *      m += (1-beta1)(g-m); v = beta2 v + (1-beta2) g^2;
 *      w = w (1 - lr wd) - lr / (1-beta1^t) * m / (sqrt(v) / sqrt(1-beta2^t) + eps).
 *   3. Muon on every block matrix (q, k, v - the three D-row blocks of wqkv, each on its own -,
 *      wo, wfc, wpr, and wtri when present): buf += (1-momentum)(g-buf);
 *      u = g + momentum (buf - g) (nesterov) or buf; X = NS(u); w -= lr_matrix * lr_mult *
 *      sqrt(max(1, rows/cols)) X, where NS is ns_steps quintic Newton-Schulz steps in bf16 on
 *      u / (||bf16(u)||_F + 1e-7): A = X X^T, B = -4.7750 A + 2.0315 A A, X = 3.4445 X + B X
 *      (tall matrices transposed), each new matrix rounded once to bf16 from fp32 accumulation.
 *   master  fp32 weights, flat layout (gpt_param_layout), updated in place.
 *   params  bf16 configurations: the bf16 copy that gpt_fwd_bwd reads, rewritten from the new
 *           master (round to nearest even); may be NULL.  fp32 configurations: NULL or master.
 *   grads   fp32 gradients, flat layout (read only; the clip factor is applied on the fly).
 *   state   fp32 [gpt_opt_state_elems]: Muon momentum of every block matrix and Adam's first
 *           moment of wte and lm_head at their flat-layout offsets, then Adam's second moments of
 *           wte and lm_head (each padded to 64 elements).  Zero it before the first step.
 *   workspace  at least gpt_opt_workspace_bytes, 256-byte aligned (Newton-Schulz buffers of one
 *           shape group, partial sums); grad_norm: fp32 device scalar (may be NULL) receiving
 *           the norm before clipping.
 * Deterministic: every reduction has a fixed order.  Stream-ordered; never synchronises. */
typedef struct {
  float lr_matrix;       /* Muon learning rate (0.02) */
  float lr_embedding;    /* Adam lr of wte before the d_model scaling (0.2) */
  float lr_unembedding;  /* Adam lr of lm_head before the d_model scaling (0.004) */
  float lr_mult;         /* schedule factor of this step, e.g. gpt_lr_multiplier */
  float momentum;        /* Muon momentum of this step, e.g. gpt_muon_momentum */
  float beta1, beta2;    /* Adam (0.8, 0.95) */
  float eps;             /* Adam (1e-10) */
  float weight_decay;    /* Adam (0) */
  float grad_clip;       /* maximum global gradient norm (1.0); 0 disables clipping */
  int32_t nesterov;      /* 1: Nesterov form of the momentum */
  int32_t ns_steps;      /* Newton-Schulz steps (5) */
  int64_t adam_step;     /* Adam steps taken including this one (1 on the first) */
} gpt_opt_hparams;

/* fp32 elements of optimizer state for cfg [host]; -1 for an invalid configuration. */
int64_t gpt_opt_state_elems(const gpt_config* cfg);
/* Device workspace in bytes for gpt_opt_step [host]. */
gpt_status gpt_opt_workspace_bytes(const gpt_config* cfg, size_t* bytes);
gpt_status gpt_opt_step(const gpt_config* cfg, float* master, void* params, const float* grads,
                        float* state, const gpt_opt_hparams* hp, void* workspace,
                        size_t ws_bytes, float* grad_norm, hipStream_t stream);
/* Schedules of the same script [host, pure]: the lr factor of iteration `it` (linear warmup over
 * round(warmup_ratio * num_iterations) iterations, then 1, then linear warmdown over the last
 * round(warmdown_ratio * num_iterations) to final_lr_frac), and Muon's momentum (0.85 rising
 * linearly to 0.95 over 300 iterations).  round() is to nearest, ties to even. */
double gpt_lr_multiplier(int64_t it, int64_t num_iterations, double warmup_ratio,
                         double warmdown_ratio, double final_lr_frac);
double gpt_muon_momentum(int64_t it);

/* ---- Inference with a key/value cache (GPT.forward with kv_cache and GPT.generate on the
 * nanochat page).  A context holds the rotary tables and, per layer, the keys (after rotary and
 * QK-norm) and values of up to max_batch sequences of max_seq positions.
 * gpt_infer_forward appends a chunk of T tokens to every sequence (cache positions p .. p+T-1,
 * p = gpt_infer_position): query p+t attends to cache positions 0 .. p+t (the page's full causal
 * pass, single query over the cache, and chunk after a prefix are its special cases).  It writes
 * the softcapped logits of each sequence's last position, fp32 [B, V], and advances the position.
 * Arguments (device pointers unless stated): params = the flat parameter buffer of
 * gpt_param_layout in cfg->dtype, 16-byte aligned; tokens = int32 [B, T] row-major (ids outside
 * [0, vocab) are clamped into it and reported by gpt_infer_check_errors, as in gpt_fwd_bwd);
 * logits = fp32 [B, V], 16-byte aligned.
 * The workspace (device, 256-byte aligned, gpt_infer_workspace_bytes) belongs to the caller and
 * must outlive the context; the context itself is host memory released by gpt_infer_destroy.
 * Work is queued on `stream` (results valid once it has run); init queues the rotary tables on
 * its stream, so work on another stream must be ordered after it by the caller.
 * Errors, with nothing queued and the position unchanged: GPT_EINVAL for null or misaligned
 * buffers and for configs with table addends (has_x0_add, has_v_add, has_trigram must be 0),
 * GPT_ESHAPE for B outside 1..max_batch or a batch size different from the one in use (it is
 * fixed from the first call until gpt_infer_reset), GPT_ERANGE when p + T > max_seq,
 * GPT_EWORKSPACE for a missing, misaligned or small workspace.  Requires max_seq <= 8192.
 * Calls on one context must not overlap (they share its buffers). */
typedef struct gpt_infer gpt_infer;
gpt_status gpt_infer_workspace_bytes(const gpt_config* cfg, int32_t max_batch, int32_t max_seq,
                                     size_t* bytes);
gpt_status gpt_infer_init(const gpt_config* cfg, int32_t max_batch, int32_t max_seq,
                          void* workspace, size_t ws_bytes, hipStream_t stream, gpt_infer** out);
gpt_status gpt_infer_reset(gpt_infer* ctx);
int32_t gpt_infer_position(const gpt_infer* ctx);
gpt_status gpt_infer_forward(gpt_infer* ctx, const void* params, const int32_t* tokens,
                             int32_t B, int32_t T, float* logits, hipStream_t stream);
/* Per-stage timing of gpt_infer_forward, as gpt_profile / gpt_profile_read for the training step:
 * with profiling on, every launch is bracketed by two events on the call's stream and tagged with
 * its stage (embed, rmsnorm, qkv, rope_append, attention or attn_split + attn_combine, out
 * [+ out_resid_norm], up, down [+ down_resid_norm], gather_last, final_norm, head, softcap) and
 * algorithmic work; the read aggregates by stage, clears the record, and fills up to *count
 * entries [host]. */
gpt_status gpt_infer_profile(gpt_infer* ctx, int32_t enable);
gpt_status gpt_infer_profile_read(gpt_infer* ctx, gpt_profile_entry* out, int32_t* count);
/* Bit flags of problems the context's kernels detected since init or the last call (1 = an input
 * id outside [0, vocab)); synchronises `stream`, then clears the flags.  flags [host]. */
gpt_status gpt_infer_check_errors(gpt_infer* ctx, hipStream_t stream, int32_t* flags);
gpt_status gpt_infer_destroy(gpt_infer* ctx);
/* Next-token choice per row of logits [B, V] fp32 (GPT.generate): temperature 0 -> argmax (the
 * first of equal maxima); otherwise logits below the top_k-th largest are dropped (top_k 0 or
 * >= V keeps all; values equal to it are kept), the rest divided by the temperature and
 * softmaxed, and the token is the first index whose cumulative probability exceeds
 * uniforms[b] (a caller-drawn number in [0, 1), the page's generator draw).  tokens int32 [B].
 * Requires V <= 65536. */
gpt_status gpt_sample(const float* logits, int32_t B, int32_t V, float temperature, int32_t top_k,
                      const float* uniforms, int32_t* tokens, hipStream_t stream);

/* Hashed n-gram gather-add (decoder-rtx bigram/trigram tables).  For each sequence b and
 * position t with current id c = tokens[b,t], previous ids p = tokens[b,t-1], pp = tokens[b,t-2]
 * (a missing previous id is `vocab`):
 *   order 2: h = (p * 1000003 + c) mod rows;  order 3: h = ((pp * 1000003 + p) * 1000003 + c) mod rows
 * in exact 64-bit integer arithmetic (ids are read as unsigned 32-bit values), then
 *   y[b*T+t, :] += table[h, :]   (fp32 add, one rounding to `dtype`).
 * tokens int32 [B,T]; table [rows, dim] and y [B*T, dim] in `dtype`; h_out int32 [B*T] or
 * NULL.  Requires dim % 8 == 0, 1 <= rows < 2^31, order in {2, 3}. */
gpt_status bigram_fwd(const int32_t* tokens, int32_t B, int32_t T, int32_t order, int32_t vocab,
                      const void* table, int64_t rows, int32_t dim, gpt_dtype dtype, void* y,
                      int32_t* h_out, hipStream_t stream);

/* Device workspace in bytes for bigram_bwd_update over n tokens of width dim [host]. */
size_t bigram_workspace_bytes(int64_t n, int32_t dim);

/* Sparse table update inlined in the tables' backward (decoder-rtx: no first moment, one
 * magnitude per row, no .grad buffer).  For every row r hit by h (rows never hit are left
 * bit-identical):
 *   g_r = sum over t with h[t] == r of dy[t, :]    (fp32, in ascending t: deterministic)
 *   v[r] = beta2 * v[r] + (1 - beta2) * mean_j g_r[j]^2
 *   table[r, :] -= lr * g_r / (sqrt(v[r]) + eps)   (uses the new v[r])
 * h int32 [n] (entries outside [0, rows) are skipped); dy [n, dim] in `dtype`; table
 * [rows, dim] in `dtype` and v fp32 [rows] updated in place.  workspace: at least
 * bigram_workspace_bytes(n, dim) bytes, 256-byte aligned.  Requires dim % 8 == 0,
 * n < 2^31.  n == 0 is a no-op. */
gpt_status bigram_bwd_update(const int32_t* h, const void* dy, int64_t n, int32_t dim,
                             gpt_dtype dtype, void* table, float* v, int64_t rows, float lr,
                             float beta2, float eps, void* workspace, size_t ws_bytes,
                             hipStream_t stream);

/* bigram_bwd_update for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same computation, kernels
 * and results, with the sort keys, histograms and edge partials in a fixed 32 MiB scratch array
 * inside the library instead of a caller workspace.  Allocates nothing (no hipMalloc, hipFree or
 * allocating library call); each GPU the library runs on holds its own copy of the array until
 * the process ends, looked up on the first call made with that GPU current.  Limit:
 * bigram_workspace_bytes(n, dim) <= 32 MiB (at dim 768 about 298,000 tokens); larger n returns
 * GPT_ESHAPE before any launch.  Every call on one GPU shares that GPU's array: calls that
 * overlap on a GPU (other streams, other host threads) race and must be ordered by the caller.
 * Arguments and errors otherwise as bigram_bwd_update. */
gpt_status bigram_bwd_update_noalloc(const int32_t* h, const void* dy, int64_t n, int32_t dim,
                                     gpt_dtype dtype, void* table, float* v, int64_t rows,
                                     float lr, float beta2, float eps, hipStream_t stream);

/* Message for the last failing call on this thread [host]; never NULL. */
const char* gpt_last_error(void);
const char* gpt_status_string(gpt_status s);

#ifdef __cplusplus
}
#endif
#endif /* GPT_H_ */
