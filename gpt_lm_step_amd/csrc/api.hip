// C ABI of libgpt: argument validation, error reporting, the flat parameter layout and the
// table entry points.  The step entry points (gpt_init, gpt_fwd_bwd, ...) live in step.hip.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>

#include "kernels.h"

namespace gpt {

static thread_local std::string g_last_error = "no error";

void set_error(const std::string& msg) { g_last_error = msg; }

gpt_status fail(gpt_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

gpt_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(GPT_EHIP, std::string(what) + ": " + hipGetErrorString(e));
  return GPT_OK;
}

gpt_status prof_read(Prof& pr, gpt_profile_entry* out, int32_t* count, const char* who) {
  std::vector<gpt_profile_entry> agg;
  for (const ProfRec& r : pr.recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(GPT_EHIP, std::string(who) + ": event sync failed");
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(GPT_EHIP, std::string(who) + ": elapsed failed");
    gpt_profile_entry* e = nullptr;
    for (auto& x : agg)
      if (strcmp(x.name, r.name) == 0) e = &x;
    if (!e) {
      agg.push_back(gpt_profile_entry{});
      e = &agg.back();
      snprintf(e->name, sizeof(e->name), "%s", r.name);
    }
    e->calls += 1;
    e->ms += ms;
    e->flops += r.flops;
    e->bytes += r.bytes;
  }
  pr.recs.clear();
  pr.next = 0;
  const int32_t cap = *count;
  *count = (int32_t)agg.size();
  if (out)
    for (int32_t i = 0; i < std::min(cap, *count); ++i) out[i] = agg[i];
  return GPT_OK;
}

// Scratch of bigram_bwd_update_noalloc: one copy per GPU, alive until the process ends.  Host
// code never passes `scratch` itself to a kernel (on the host it names a stand-in, not device
// memory); it uses the device address hipGetSymbolAddress gives for the current device, looked up
// once per device on that device's first call and kept here.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];
constexpr int NOALLOC_MAX_DEVICES = 64;
static void* g_scratch_ptr[NOALLOC_MAX_DEVICES];
static std::mutex g_scratch_mu;

static gpt_status scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES)
    return fail(GPT_EHIP, "bigram_bwd_update_noalloc: no usable current device");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(GPT_EHIP, std::string("bigram_bwd_update_noalloc: hipGetSymbolAddress: ") +
                                hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return GPT_OK;
}

}  // namespace gpt

using namespace gpt;

extern "C" {

const char* gpt_last_error(void) { return g_last_error.c_str(); }

const char* gpt_status_string(gpt_status s) {
  switch (s) {
    case GPT_OK: return "ok";
    case GPT_EINVAL: return "invalid argument";
    case GPT_ESHAPE: return "unsupported shape";
    case GPT_ERANGE: return "value out of range";
    case GPT_EWORKSPACE: return "workspace too small";
    case GPT_EHIP: return "HIP error";
  }
  return "unknown status";
}

gpt_status bigram_fwd(const int32_t* tokens, int32_t B, int32_t T, int32_t order, int32_t vocab,
                      const void* table, int64_t rows, int32_t dim, gpt_dtype dtype, void* y,
                      int32_t* h_out, hipStream_t stream) {
  if (B < 0 || T < 0) return fail(GPT_ESHAPE, "bigram_fwd: negative B or T");
  if ((long long)B * T == 0) return GPT_OK;
  if (!tokens || !table || !y) return fail(GPT_EINVAL, "bigram_fwd: null pointer");
  if (order != 2 && order != 3) return fail(GPT_EINVAL, "bigram_fwd: order must be 2 or 3");
  if (vocab < 0) return fail(GPT_ERANGE, "bigram_fwd: negative vocab");
  if (rows < 1 || rows >= (1LL << 31)) return fail(GPT_ERANGE, "bigram_fwd: rows out of range");
  if (dim <= 0 || dim % 8) return fail(GPT_ESHAPE, "bigram_fwd: dim must be a positive multiple of 8");
  if (dtype == GPT_BF16)
    return launch_bigram_fwd<bf16>(tokens, B, T, order, vocab, (const bf16*)table, rows, dim,
                                   (bf16*)y, h_out, stream);
  if (dtype == GPT_F32)
    return launch_bigram_fwd<float>(tokens, B, T, order, vocab, (const float*)table, rows, dim,
                                    (float*)y, h_out, stream);
  return fail(GPT_EINVAL, "bigram_fwd: bad dtype");
}

size_t bigram_workspace_bytes(int64_t n, int32_t dim) {
  if (n <= 0 || dim <= 0) return 0;
  return segsum_workspace_bytes(n, dim);
}

gpt_status bigram_bwd_update(const int32_t* h, const void* dy, int64_t n, int32_t dim,
                             gpt_dtype dtype, void* table, float* v, int64_t rows, float lr,
                             float beta2, float eps, void* workspace, size_t ws_bytes,
                             hipStream_t stream) {
  if (n < 0 || n >= (1LL << 31)) return fail(GPT_ESHAPE, "bigram_bwd_update: n out of range");
  if (n == 0) return GPT_OK;
  if (!h || !dy || !table || !v) return fail(GPT_EINVAL, "bigram_bwd_update: null pointer");
  if (dim <= 0 || dim % 8 || dim > 2048)
    return fail(GPT_ESHAPE, "bigram_bwd_update: dim must be a multiple of 8 in [8, 2048]");
  if (rows < 1 || rows >= (1LL << 31)) return fail(GPT_ERANGE, "bigram_bwd_update: rows out of range");
  if (!workspace || ws_bytes < bigram_workspace_bytes(n, dim))
    return fail(GPT_EWORKSPACE, "bigram_bwd_update: workspace too small");
  if (((uintptr_t)workspace) % 256) return fail(GPT_EINVAL, "bigram_bwd_update: workspace not 256-byte aligned");
  if (dtype == GPT_BF16)
    return segsum_update<bf16>(h, (const bf16*)dy, n, dim, (bf16*)table, v, rows, lr, beta2, eps,
                               workspace, ws_bytes, stream);
  if (dtype == GPT_F32)
    return segsum_update<float>(h, (const float*)dy, n, dim, (float*)table, v, rows, lr, beta2,
                                eps, workspace, ws_bytes, stream);
  return fail(GPT_EINVAL, "bigram_bwd_update: bad dtype");
}

gpt_status bigram_bwd_update_noalloc(const int32_t* h, const void* dy, int64_t n, int32_t dim,
                                     gpt_dtype dtype, void* table, float* v, int64_t rows,
                                     float lr, float beta2, float eps, hipStream_t stream) {
  if (n < 0 || n >= (1LL << 31)) return fail(GPT_ESHAPE, "bigram_bwd_update_noalloc: n out of range");
  if (n == 0) return GPT_OK;
  if (dim <= 0 || dim % 8 || dim > 2048)
    return fail(GPT_ESHAPE, "bigram_bwd_update_noalloc: dim must be a multiple of 8 in [8, 2048]");
  const size_t need = bigram_workspace_bytes(n, dim);
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(GPT_ESHAPE, "bigram_bwd_update_noalloc: n = " + std::to_string(n) + ", dim = " +
                                std::to_string(dim) + " needs " + std::to_string(need) +
                                " bytes of scratch, above its fixed " +
                                std::to_string(NOALLOC_SCRATCH_BYTES) + " (use bigram_bwd_update)");
  void* ws = nullptr;
  gpt_status st = scratch_for_current_device(&ws);
  if (st != GPT_OK) return st;
  // Nothing in the scratch has to start at zero: every pass writes what later passes read.
  return bigram_bwd_update(h, dy, n, dim, dtype, table, v, rows, lr, beta2, eps, ws,
                           NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
