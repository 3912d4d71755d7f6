// Host-side launchers of the gfx950 kernels (internal to libgpt; not part of the ABI).
#pragma once

#include <string>
#include <vector>

#include "common.h"

namespace gpt {

// ---------------------------------------------------------------- parameter layout (step.hip)
// Offsets (elements) of every tensor of the flat parameter / gradient buffer, in the order of
// gpt_param_layout, each a multiple of PARAM_ALIGN.
constexpr int PARAM_ALIGN = 64;
inline long long align_elems(long long n) { return (n + PARAM_ALIGN - 1) / PARAM_ALIGN * PARAM_ALIGN; }
struct Layout {
  struct Entry {
    std::string name;
    long long off, rows, cols;
  };
  std::vector<Entry> e;
  long long total = 0;
  long long wte, lm_head, wtri = -1;
  std::vector<long long> wqkv, wo, wfc, wpr;
};
Layout make_layout(const gpt_config& c);
// Argument checks shared by every entry point that takes a configuration.
gpt_status validate(const gpt_config* c);

// ---------------------------------------------------------------- tables / segments
// Hash + gather-add of one n-gram table (bigram_fwd).
template <typename T>
gpt_status launch_bigram_fwd(const int32_t* tokens, int B, int T_, int order, int vocab,
                             const T* table, long long rows, int dim, T* y, int32_t* h_out,
                             hipStream_t s);

// Scratch for the sort + segmented reduction over n keys of width dim.
size_t segsum_workspace_bytes(long long n, int dim);

// Sparse per-row update of `table`/`v` from per-token grads dy (bigram_bwd_update).
template <typename T>
gpt_status segsum_update(const int32_t* keys, const T* dy, long long n, int dim, T* table,
                         float* v, long long rows, float lr, float beta2, float eps, void* ws,
                         size_t ws_bytes, hipStream_t s);

// Dense fp32 gradient out[row] = beta * out[row] + sum of dy rows whose key is row.  Rows no
// key hits are untouched (the caller zeroes them when beta == 0).
gpt_status segsum_grad(const int32_t* keys, const float* dy, long long n, int dim, float* out,
                       long long rows, int beta, void* ws, size_t ws_bytes, hipStream_t s);

// ---------------------------------------------------------------- rows / norms (norm.hip)
template <typename T>
gpt_status launch_rope_table(T* cos_t, T* sin_t, int Tn, int hd, float base, hipStream_t s);
template <typename T>
gpt_status launch_embed_fwd(const int32_t* tok, const T* wte, const T* x0_add, float* x,
                            float* rstd, int32_t* tok_c, int* err, long long N, int D, int V,
                            float eps, hipStream_t s);
template <typename T>
gpt_status launch_embed_bwd(const int32_t* tok_c, const T* wte, const float* rstd,
                            const float* dx, float* de, long long N, int D, hipStream_t s);
template <typename T>
gpt_status launch_rms_fwd(const float* x, T* y, float* rstd, long long N, int D, float eps,
                          hipStream_t s);
template <typename T>
gpt_status launch_rms_bwd(const float* x, const float* rstd, const float* dy, const float* dres,
                          float* dx, T* dx_t, long long N, int D, hipStream_t s);
template <typename T>
gpt_status launch_rope_qknorm_fwd(T* qkv, const T* cos_t, const T* sin_t, float* rstd_qk,
                                  long long N, int Tn, int H, int hd, int qk_norm, float eps,
                                  hipStream_t s);
template <typename T>
gpt_status launch_rope_qknorm_bwd(T* dqkv, const T* qkv, const T* cos_t, const T* sin_t,
                                  const float* rstd_qk, long long N, int Tn, int H, int hd,
                                  int qk_norm, hipStream_t s);
gpt_status launch_fill(float* p, long long n, float v, hipStream_t s);
// Workspace guards (Carver): check == 0 writes GUARD_WORD over the n guards listed in tab
// (byte offsets into ws); check == 1 sets bit 4 of *err if any guard word differs.
gpt_status launch_guards(char* ws, const long long* tab, int n, int* err, int check,
                         hipStream_t s);
template <typename T>
gpt_status launch_accum_rows(float* dst, const T* src, long long lds, long long N, int D, int add,
                             hipStream_t s);
template <typename T>
gpt_status launch_cast(T* dst, const float* src, long long n, hipStream_t s);

// ---------------------------------------------------------------- cross-entropy (ce.hip)
gpt_status launch_count_targets(const int32_t* tgt, long long N, int V, int* n_valid, int* err,
                                hipStream_t s);
template <typename T>
gpt_status launch_ce(T* z, long long ldz, const int32_t* tgt, long long rows, int V, float cap,
                     float grad_scale, const int* n_valid, float* loss_rows, hipStream_t s);
gpt_status launch_loss_reduce(const float* loss_rows, long long N, const int* n_valid,
                              float* loss, hipStream_t s);

// ---------------------------------------------------------------- attention (attn.hip)
// qk_normed: q and k are RMS-normalized per head (the QK-norm), which bounds every score, so
// the softmax needs no running maximum.
template <typename T>
gpt_status launch_attn_fwd(const T* qkv, T* out, float* lse2, int B, int Tn, int H, int hd,
                           hipStream_t s, int qk_normed = 0);
// stage 0: rowsum(dO * O) into dq_sum and dQ; stage 1: dK, dV (reads dq_sum).
template <typename T>
gpt_status launch_attn_bwd_stage(int stage, const T* qkv, const T* out, const T* dout,
                                 const float* lse2, float* dq_sum, T* dqkv, int B, int Tn, int H,
                                 int hd, hipStream_t s);
template <typename T>
gpt_status launch_attn_bwd(const T* qkv, const T* out, const T* dout, const float* lse2,
                           float* dq_sum, T* dqkv, int B, int Tn, int H, int hd, hipStream_t s);

// Optional per-launch timing: when enabled, every launch of a step is bracketed by two events
// on the step's stream and tagged with its stage name and algorithmic work.
struct ProfRec {
  const char* name;
  double flops, bytes;
  hipEvent_t a, b;
};
struct Prof {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  size_t next = 0;
  hipEvent_t get() {
    if (next == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      pool.push_back(e);
    }
    return pool[next++];
  }
  ~Prof() {
    for (hipEvent_t e : pool) (void)hipEventDestroy(e);
  }
};

// Aggregates the recorded launches by stage name (in order of first launch) after waiting for
// their events, clears the record, and writes up to *count entries (*count: capacity in, number
// of stages out; out may be null).  `who` names the entry point in error messages.
gpt_status prof_read(Prof& pr, gpt_profile_entry* out, int32_t* count, const char* who);

}  // namespace gpt
