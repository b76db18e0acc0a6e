// Host-side contract of the C ABI (include/ttt.h, include/ttt_kernels.h) for a
// build of the library's host code with AddressSanitizer (tests/test_sanitizers.py):
// argument validation, configuration errors, the allocator hook, error messages
// and every call on a NULL context.  Needs no GPU: a valid configuration on a
// machine without a gfx950 device must give TTT_ENODEV and leave nothing
// allocated.  Exit status 0 when every call returned what it should.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "ttt.h"
#include "ttt_kernels.h"

static int failures = 0;
#define CHECK(cond)                                                                 \
  do {                                                                              \
    if (!(cond)) {                                                                  \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);       \
      ++failures;                                                                   \
    }                                                                               \
  } while (0)

namespace {

constexpr int L = 2, D = 16, H = 2, F = 24, V = 11;

struct Weights {
  std::vector<float> embed = std::vector<float>(V * D, 0.01f), final_norm = std::vector<float>(D, 1.f),
                     lm_head = std::vector<float>(V * D, 0.01f);
  std::vector<std::vector<float>> per[9];
  const float* ptrs[9][L];
  ttt_weights w{};
  Weights() {
    const size_t sizes[9] = {D, D * D, D * D, D * D, D * D, D, F * D, F * D, D * F};
    for (int a = 0; a < 9; ++a)
      for (int l = 0; l < L; ++l) {
        per[a].emplace_back(sizes[a], (a == 0 || a == 5) ? 1.f : 0.02f);
        ptrs[a][l] = per[a].back().data();
      }
    w.embed = embed.data();
    w.final_norm = final_norm.data();
    w.lm_head = lm_head.data();
    w.attn_norm = ptrs[0];
    w.wq = ptrs[1];
    w.wk = ptrs[2];
    w.wv = ptrs[3];
    w.wo = ptrs[4];
    w.mlp_norm = ptrs[5];
    w.w_gate = ptrs[6];
    w.w_up = ptrs[7];
    w.w_down = ptrs[8];
  }
};

ttt_config good_cfg() {
  ttt_config c{};
  c.n_layers = L;
  c.d_model = D;
  c.n_heads = H;
  c.d_ff = F;
  c.vocab = V;
  c.window = 8;
  c.chunk = 4;
  c.n_fast = 0;
  c.batch = 1;
  c.dtype = TTT_F32;
  c.max_positions = 64;
  c.rope_theta = 1e4;
  c.rms_eps = 1e-5;
  c.lr = 0.1f;
  return c;
}

int create_rc(const ttt_config& c, const Weights& w, std::string* msg) {
  ttt_ctx* h = reinterpret_cast<ttt_ctx*>(0x1);
  const int rc = ttt_create(&c, &w.w, nullptr, &h);
  if (msg) *msg = ttt_last_error(nullptr);
  if (rc == TTT_OK) {
    ttt_destroy(h);
  } else {
    CHECK(h == nullptr);
  }
  return rc;
}

int hook_calls = 0;
void* hook_alloc(size_t, void*) {
  ++hook_calls;
  return nullptr;
}
void hook_free(void*, void*) {}

}  // namespace

int main() {
  Weights w;
  std::string msg;

  // NULL arguments
  ttt_ctx* h = nullptr;
  ttt_config c = good_cfg();
  CHECK(ttt_create(nullptr, &w.w, nullptr, &h) == TTT_EINVAL);
  CHECK(ttt_create(&c, nullptr, nullptr, &h) == TTT_EINVAL);
  CHECK(ttt_create(&c, &w.w, nullptr, nullptr) == TTT_EINVAL);
  CHECK(std::strlen(ttt_last_error(nullptr)) > 0);

  // invalid configurations: each is refused before any device query
  struct Bad {
    void (*edit)(ttt_config&);
    const char* word;
  } bads[] = {
      {[](ttt_config& x) { x.window = 3; }, "window"},
      {[](ttt_config& x) { x.chunk = 0; }, "window"},
      {[](ttt_config& x) { x.d_model = 15; }, "multiple"},
      {[](ttt_config& x) { x.n_fast = 3; }, "n_fast"},
      {[](ttt_config& x) { x.max_positions = 0; }, "max_positions"},
      {[](ttt_config& x) { x.lr = NAN; }, "lr"},
      {[](ttt_config& x) { x.dtype = 7; }, "dtype"},
      {[](ttt_config& x) { x.batch = 0; }, "positive"},
      {[](ttt_config& x) { x.n_steps = -1; }, "n_steps"},
  };
  for (const Bad& b : bads) {
    ttt_config x = good_cfg();
    b.edit(x);
    CHECK(create_rc(x, w, &msg) == TTT_EINVAL);
    if (msg.find(b.word) == std::string::npos) {
      std::fprintf(stderr, "message for '%s' case: %s\n", b.word, msg.c_str());
      ++failures;
    }
  }

  // a NULL weight array is refused too, and so is the dual MLP without its dynamic weights
  Weights w2;
  w2.w.wq = nullptr;
  CHECK(create_rc(good_cfg(), w2, &msg) == TTT_EINVAL);
  ttt_config cd = good_cfg();
  cd.dual_mlp = 1;
  CHECK(create_rc(cd, w, &msg) == TTT_EINVAL && msg.find("dyn_") != std::string::npos);
  cd.dual_mlp = 2;
  CHECK(create_rc(cd, w, &msg) == TTT_EINVAL && msg.find("dual_mlp") != std::string::npos);

  // allocator hook: both or neither
  CHECK(ttt_set_allocator(hook_alloc, nullptr, nullptr) == TTT_EINVAL);
  CHECK(ttt_set_allocator(hook_alloc, hook_free, nullptr) == TTT_OK);
  const int rc_hook = create_rc(good_cfg(), w, &msg);
  CHECK(rc_hook == TTT_ENODEV || rc_hook == TTT_ENOMEM);
  CHECK(ttt_set_allocator(nullptr, nullptr, nullptr) == TTT_OK);

  // a valid configuration without a device
  const int rc = create_rc(good_cfg(), w, &msg);
  CHECK(rc == TTT_ENODEV);

  // every call on a NULL context
  int32_t ids[4] = {0, 1, 2, 3};
  float f4[4] = {0, 0, 0, 0};
  double ms[TTT_PROF_CLASSES], fl[TTT_PROF_CLASSES];
  int64_t cnt[TTT_PROF_CLASSES];
  CHECK(ttt_prefill_chunk(nullptr, ids, ids, 4, f4) == TTT_EINVAL);
  CHECK(ttt_prefill(nullptr, ids, ids, 4, f4) == TTT_EINVAL);
  CHECK(ttt_prefill_device(nullptr, ids, ids, 4, f4) == TTT_EINVAL);
  CHECK(ttt_score(nullptr, ids, ids, 4, f4) == TTT_EINVAL);
  CHECK(ttt_score_device(nullptr, ids, ids, 4, f4) == TTT_EINVAL);
  CHECK(ttt_sync(nullptr) == TTT_EINVAL);
  CHECK(ttt_generate(nullptr, ids, 4, 4, ids, f4) == TTT_EINVAL);
  CHECK(ttt_get_fast_weights(nullptr, 0, f4, 4) == TTT_EINVAL);
  CHECK(ttt_set_fast_weights(nullptr, 0, f4, 4) == TTT_EINVAL);
  CHECK(ttt_state_size(nullptr) < 0);
  CHECK(ttt_save_state(nullptr, f4, 16) == TTT_EINVAL);
  CHECK(ttt_load_state(nullptr, f4, 16) == TTT_EINVAL);
  CHECK(ttt_reset(nullptr) == TTT_EINVAL);
  CHECK(ttt_position(nullptr) == -1);
  CHECK(ttt_profile_enable(nullptr, -1) == TTT_EINVAL);
  CHECK(ttt_profile_read(nullptr, TTT_PROF_CLASSES, ms, cnt, fl) == TTT_EINVAL);
  ttt_destroy(nullptr);

  // kernel entry points: argument errors come back before any launch
  float buf[64];
  CHECK(tttk_gemm(TTT_F32, nullptr, 8, buf, 8, buf, 8, 1, 1, 8, nullptr, 0, nullptr) == TTT_EINVAL);
  CHECK(tttk_gemm(TTT_F32, buf, 4, buf, 8, buf, 8, 1, 1, 8, nullptr, 0, nullptr) == TTT_EINVAL);
  CHECK(tttk_gemm(9, buf, 8, buf, 8, buf, 8, 1, 1, 8, nullptr, 0, nullptr) != TTT_OK);
  CHECK(tttk_swa_fwd(TTT_F32, buf, buf, buf, buf, buf, nullptr, 1, 1, 3, 1, 8, 4, 0, nullptr, 0, nullptr) ==
        TTT_EINVAL);  // odd head_dim
  CHECK(tttk_swa_fwd(TTT_F32, buf, buf, buf, buf, buf, nullptr, 1, 1, 4, 4, 5, 4, 0, nullptr, 0, nullptr) ==
        TTT_EINVAL);  // ring shorter than window + n - 1
  CHECK(tttk_swa_fwd_noalloc(TTT_BF16, nullptr, buf, buf, buf, buf, nullptr, 1, 1, 4, 1, 8, 4, 0, nullptr) ==
        TTT_EINVAL);
  CHECK(tttk_swa_bwd(TTT_F32, buf, buf, buf, buf, buf, nullptr, buf, buf, buf, buf, buf, buf, buf, nullptr, 1, 1, 4,
                     4, 8, 2, 0, nullptr, 0, nullptr) == TTT_EINVAL);  // window < n

  if (failures) {
    std::fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  std::printf("abi driver: all checks passed\n");
  return 0;
}
