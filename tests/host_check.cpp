// Host-side check of libgpt's C ABI, built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host code (tests/test_host_sanitizers.py).  It drives every path that runs without a
// GPU: parameter layouts, workspace planning (the carve of every buffer of a step, an optimizer
// step and an inference context), schedules, and the argument checks that reject a call before
// any launch.  A sanitizer report or a wrong status fails the run.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gpt.h"
#include "gpt_kernels.h"

static int failures = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                       \
    }                                                                   \
  } while (0)

static gpt_config make(int L, int D, int H, int hd, int F, int V, int T, int B, int dtype,
                       int x0, int va, int tri) {
  gpt_config c;
  std::memset(&c, 0, sizeof(c));
  c.n_layer = L; c.d_model = D; c.n_head = H; c.n_kv_head = H; c.head_dim = hd; c.d_mlp = F;
  c.vocab = V; c.seq_len = T; c.batch = B; c.dtype = dtype; c.rms_eps = 1e-6f;
  c.rope_base = 10000.f; c.softcap = 15.f; c.qk_norm = 1;
  c.has_x0_add = x0; c.has_v_add = va; c.has_trigram = tri;
  return c;
}

int main() {
  std::vector<gpt_config> cfgs = {
      make(2, 128, 4, 32, 512, 512, 64, 4, GPT_F32, 0, 0, 0),        // tiny
      make(2, 128, 4, 32, 512, 512, 64, 4, GPT_F32, 1, 1, 1),        // tiny + tables
      make(12, 768, 12, 64, 3072, 50304, 1024, 8, GPT_BF16, 0, 0, 0),  // GPT-2-small
      make(12, 768, 12, 64, 3072, 50304, 1024, 8, GPT_BF16, 1, 1, 1),  // speedrun
      make(32, 2048, 16, 128, 8192, 65536, 2048, 8, GPT_BF16, 0, 0, 0),  // d32
  };
  for (gpt_config c : cfgs) {
    int32_t count = 0;
    int64_t total = 0;
    CHECK(gpt_param_layout(&c, nullptr, &count, &total) == GPT_OK);
    std::vector<gpt_tensor_desc> d(count);
    int32_t cap = count;
    CHECK(gpt_param_layout(&c, d.data(), &cap, &total) == GPT_OK && cap == count);
    for (int32_t i = 1; i < count; ++i) CHECK(d[i].offset_elems >= d[i - 1].offset_elems);
    CHECK(std::strlen(d[count - 1].name) > 0);
    int32_t small = count - 1;
    if (count > 1) CHECK(gpt_param_layout(&c, d.data(), &small, &total) == GPT_EINVAL);
    size_t ws = 0;
    CHECK(gpt_workspace_bytes(&c, &ws) == GPT_OK && ws > 0);
    for (int chunk : {64, 192, 4096}) {
      gpt_config cc = c;
      cc.ce_chunk_tokens = chunk;
      size_t w2 = 0;
      CHECK(gpt_workspace_bytes(&cc, &w2) == GPT_OK && w2 <= ws);
    }
    CHECK(gpt_opt_state_elems(&c) > 0);
    size_t ow = 0;
    CHECK(gpt_opt_workspace_bytes(&c, &ow) == GPT_OK);
    if (!c.has_x0_add) {
      size_t iw = 0;
      CHECK(gpt_infer_workspace_bytes(&c, 8, 2048, &iw) == GPT_OK && iw > 0);
      CHECK(gpt_infer_workspace_bytes(&c, 0, 2048, &iw) != GPT_OK);
    }
    // init over a fake, aligned address that is too small, and misaligned: rejected before use
    gpt_ctx* ctx = nullptr;
    CHECK(gpt_init(&c, reinterpret_cast<void*>(uintptr_t(1) << 20), 1024, nullptr, &ctx) == GPT_EWORKSPACE);
    CHECK(gpt_init(&c, reinterpret_cast<void*>((uintptr_t(1) << 20) + 8), ws, nullptr, &ctx) == GPT_EINVAL);
    CHECK(gpt_init(&c, nullptr, ws, nullptr, &ctx) == GPT_EWORKSPACE);
  }
  // invalid configurations
  {
    gpt_config c = cfgs[0];
    size_t ws = 0;
    gpt_config b = c; b.head_dim = 48; b.n_head = 1; b.d_model = 48;
    CHECK(gpt_workspace_bytes(&b, &ws) == GPT_ESHAPE);
    b = c; b.vocab = 500; CHECK(gpt_workspace_bytes(&b, &ws) == GPT_ESHAPE);
    b = c; b.seq_len = 100; CHECK(gpt_workspace_bytes(&b, &ws) == GPT_ESHAPE);
    b = c; b.dtype = 7; CHECK(gpt_workspace_bytes(&b, &ws) == GPT_EINVAL);
    b = c; b.ce_chunk_tokens = 100; CHECK(gpt_workspace_bytes(&b, &ws) == GPT_ESHAPE);
    b = c; b.n_kv_head = 2; CHECK(gpt_workspace_bytes(&b, &ws) == GPT_ESHAPE);
    b = c; b.rms_eps = -1.f; CHECK(gpt_workspace_bytes(&b, &ws) == GPT_ERANGE);
    CHECK(gpt_workspace_bytes(nullptr, &ws) == GPT_EINVAL);
    CHECK(std::strlen(gpt_last_error()) > 0);
    for (int s = 0; s >= -5; --s) CHECK(gpt_status_string((gpt_status)s) != nullptr);
  }
  // schedules
  CHECK(gpt_lr_multiplier(0, 1000, 0.0, 0.2, 0.0) == 1.0);
  CHECK(gpt_lr_multiplier(999, 1000, 0.0, 0.2, 0.0) < 0.01);
  CHECK(gpt_muon_momentum(0) == 0.85);
  CHECK(gpt_muon_momentum(300) == 0.95);
  // table entry points: sizes and argument checks
  CHECK(bigram_workspace_bytes(0, 768) == 0);
  CHECK(bigram_workspace_bytes(196608, 768) > 0);
  CHECK(bigram_fwd(nullptr, 2, 8, 2, 100, nullptr, 16, 64, GPT_BF16, nullptr, nullptr, nullptr) == GPT_EINVAL);
  CHECK(bigram_bwd_update(nullptr, nullptr, 10, 64, GPT_BF16, nullptr, nullptr, 16, 0.1f, 0.95f,
                          1e-8f, nullptr, 0, nullptr) == GPT_EINVAL);
  CHECK(bigram_bwd_update(nullptr, nullptr, 0, 64, GPT_BF16, nullptr, nullptr, 16, 0.1f, 0.95f,
                          1e-8f, nullptr, 0, nullptr) == GPT_OK);
  CHECK(bigram_bwd_update_noalloc(nullptr, nullptr, 400000, 768, GPT_BF16, nullptr, nullptr, 16,
                                  0.1f, 0.95f, 1e-8f, nullptr) == GPT_ESHAPE);
  // per-kernel entry points: rejected before any launch
  CHECK(gptk_gemm(GPT_BF16, 1, 1, 64, 64, 64, nullptr, 64, nullptr, 64, nullptr, 64, 0, nullptr) == GPT_EINVAL);
  CHECK(gptk_gemm_wgrad_ws_floats(2048, 2048, 16384) > 0);
  CHECK(gptk_gemm_wgrad_ws_floats(0, 2048, 16384) == 0);
  CHECK(gptk_rmsnorm_fwd(GPT_BF16, nullptr, nullptr, nullptr, 10, 64, 1e-6f, nullptr) == GPT_EINVAL);
  CHECK(gptk_attention_fwd(GPT_BF16, nullptr, nullptr, nullptr, 1, 64, 2, 64, nullptr) == GPT_EINVAL);
  CHECK(gptk_softcap_ce(GPT_BF16, nullptr, 64, nullptr, 4, 64, 15.f, 1.f, nullptr, nullptr, nullptr) == GPT_EINVAL);
  CHECK(gpt_sample(nullptr, 2, 64, 1.f, 0, nullptr, nullptr, nullptr) != GPT_OK);
  CHECK(gpt_destroy(nullptr) == GPT_OK);
  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("host checks passed\n");
  return 0;
}
