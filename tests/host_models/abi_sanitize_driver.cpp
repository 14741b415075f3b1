// Drives the host side of the C ABI (argument and shape checks, packed sizes,
// error reporting, the calls' behaviour without a GPU) with the library's host
// code built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  No kernel is launched: on a machine without a
// GPU every call that needs a device must fail with an error code, not crash.
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/mk.h"

static int g_fail = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::fprintf(stderr, "FAIL %s:%d %s\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

static mk_layer_config cfg(int d, int nh, int dh, int dc, int dr, int E, int topk, int nsh, int f, int af, int ef,
                           int kf) {
  mk_layer_config c;
  std::memset(&c, 0, sizeof c);
  c.abi_version = MK_ABI_VERSION;
  c.d_model = d; c.n_heads = nh; c.d_head = dh; c.d_latent = dc; c.d_rope = dr; c.n_experts = E;
  c.top_k = topk; c.n_shared = nsh; c.d_ff = f; c.attn_format = af; c.expert_format = ef; c.kv_format = kf;
  c.rms_eps = 1e-6f; c.rope_base = 10000.f;
  return c;
}

int main() {
  CHECK(mk_abi_version() == MK_ABI_VERSION);
  CHECK(mk_last_error() != nullptr);
  const mk_layer_config good[] = {
      cfg(512, 8, 64, 128, 32, 16, 2, 1, 256, MK_FMT_F32, MK_FMT_F32, MK_FMT_F32),
      cfg(4096, 32, 128, 512, 64, 128, 8, 1, 1024, MK_FMT_BF16, MK_FMT_BF16, MK_FMT_BF16),
      cfg(4096, 32, 128, 512, 64, 384, 8, 1, 2048, MK_FMT_BF16, MK_FMT_FP8_B128, MK_FMT_BF16),
      cfg(4096, 32, 128, 512, 64, 384, 8, 1, 2048, MK_FMT_BF16, MK_FMT_MXFP4, MK_FMT_BF16),
      cfg(640, 6, 64, 256, 64, 48, 6, 1, 384, MK_FMT_BF16, MK_FMT_MXFP4, MK_FMT_BF16),
      cfg(4096, 32, 128, 512, 64, 384, 8, 1, 2048, MK_FMT_BF16, MK_FMT_MXFP4, MK_FMT_FP8_ROW),
      cfg(640, 6, 64, 256, 64, 48, 6, 1, 384, MK_FMT_BF16, MK_FMT_BF16, MK_FMT_FP8_ROW),
  };
  for (const auto& c : good) {
    CHECK(mk_check_config(&c) == MK_OK);
    for (int t = MK_T_WQ; t <= MK_T_EXPERT; ++t) {
      size_t b = 0;
      CHECK(mk_packed_bytes(&c, t, &b) == MK_OK);
      CHECK(b > 0 && b % 256 == 0);
    }
    size_t b = 0;
    CHECK(mk_packed_bytes(&c, 99, &b) == MK_ERR_INVALID_ARG);
    CHECK(mk_packed_bytes(&c, MK_T_WQ, nullptr) == MK_ERR_INVALID_ARG);
    const size_t row = c.kv_format == MK_FMT_FP8_ROW ? (size_t)(c.d_latent + c.d_rope + 4 + 15) / 16 * 16
                                                     : (size_t)(c.d_latent + c.d_rope) * (c.kv_format == MK_FMT_F32 ? 4 : 2);
    CHECK(mk_kv_bytes(&c, 8192, &b) == MK_OK && b == 8192 * row);
    CHECK(mk_kv_bytes(&c, -1, &b) == MK_ERR_INVALID_ARG);
    // without a GPU the device-dependent sizes are an error, not a crash
    CHECK(mk_layer_state_bytes(&c, 0, &b) != MK_OK);
    CHECK(mk_layer_workspace_bytes(&c, 0, &b) != MK_OK);
    CHECK(mk_layer_state_bytes(&c, 0, nullptr) == MK_ERR_INVALID_ARG);
  }
  // every kind of bad config is refused with its code
  std::vector<std::pair<mk_layer_config, int>> bad;
  mk_layer_config c = good[2];
  c.abi_version = 99; bad.push_back({c, MK_ERR_ABI_MISMATCH});
  c = good[2]; c.d_model = 0; bad.push_back({c, MK_ERR_INVALID_ARG});
  c = good[2]; c.n_heads = -3; bad.push_back({c, MK_ERR_INVALID_ARG});
  c = good[2]; c.expert_format = 7; bad.push_back({c, MK_ERR_INVALID_ARG});
  c = good[2]; c.kv_format = -1; bad.push_back({c, MK_ERR_INVALID_ARG});
  c = good[2]; c.kv_format = MK_FMT_FP8_B128; bad.push_back({c, MK_ERR_INVALID_ARG});
  c = good[0]; c.kv_format = MK_FMT_FP8_ROW; bad.push_back({c, MK_ERR_UNSUPPORTED_SHAPE});
  c = good[2]; c.has_router_bias = 2; bad.push_back({c, MK_ERR_INVALID_ARG});
  c = good[2]; c.rms_eps = -1.f; bad.push_back({c, MK_ERR_INVALID_ARG});
  c = good[2]; c.d_model = 4000; bad.push_back({c, MK_ERR_UNSUPPORTED_SHAPE});
  c = good[2]; c.n_experts = 100; bad.push_back({c, MK_ERR_UNSUPPORTED_SHAPE});
  c = good[2]; c.top_k = 17; bad.push_back({c, MK_ERR_UNSUPPORTED_SHAPE});
  c = good[2]; c.n_shared = 2; bad.push_back({c, MK_ERR_UNSUPPORTED_SHAPE});
  c = good[2]; c.attn_format = MK_FMT_F32; bad.push_back({c, MK_ERR_UNSUPPORTED_SHAPE});
  c = good[2]; c.n_experts = 2048; bad.push_back({c, MK_ERR_UNSUPPORTED_SHAPE});
  c = good[0]; c.d_latent = 512; bad.push_back({c, MK_ERR_UNSUPPORTED_SHAPE});
  for (const auto& p : bad) {
    CHECK(mk_check_config(&p.first) == p.second);
    CHECK(std::strlen(mk_last_error()) > 0);
    size_t b = 0;
    CHECK(mk_packed_bytes(&p.first, MK_T_EXPERT, &b) == p.second);
  }
  CHECK(mk_check_config(nullptr) == MK_ERR_INVALID_ARG);
  // null arguments everywhere
  size_t b = 0;
  CHECK(mk_head_packed_bytes(129280, 4096, &b) == MK_OK && b == (size_t)129280 * 4096 * 2);
  CHECK(mk_head_packed_bytes(100, 4096, &b) == MK_ERR_INVALID_ARG);
  CHECK(mk_head_packed_bytes(128, 4096, nullptr) == MK_ERR_INVALID_ARG);
  mk_device_info di;
  CHECK(mk_query_device(0, nullptr) == MK_ERR_INVALID_ARG);
  CHECK(mk_query_device(-1, &di) != MK_OK);
  mk_layer* L = nullptr;
  CHECK(mk_layer_init(&good[2], nullptr, nullptr, nullptr, 0, &L) != MK_OK && L == nullptr);
  CHECK(mk_layer_init(&good[2], nullptr, nullptr, nullptr, 0, nullptr) == MK_ERR_INVALID_ARG);
  mk_kv_cache kv = {nullptr, 0, 0};
  CHECK(mk_decode_step(nullptr, nullptr, 1, &kv, nullptr, nullptr) == MK_ERR_INVALID_ARG);
  CHECK(mk_decode_step_static(nullptr, nullptr, 1, &kv, nullptr, nullptr) == MK_ERR_INVALID_ARG);
  CHECK(mk_debug_tap(nullptr, 0, nullptr, 0, nullptr) == MK_ERR_INVALID_ARG);
  mk_stats st;
  CHECK(mk_get_stats(nullptr, &st) == MK_ERR_INVALID_ARG);
  CHECK(mk_set_trace(nullptr, 1) == MK_ERR_INVALID_ARG);
  CHECK(mk_read_trace(nullptr, nullptr, 0, nullptr) == MK_ERR_INVALID_ARG);
  CHECK(mk_set_barrier_timeout_us(nullptr, 10) == MK_ERR_INVALID_ARG);
  CHECK(mk_sync_status(nullptr) == MK_ERR_INVALID_ARG);
  CHECK(mk_layer_reset(nullptr) == MK_ERR_INVALID_ARG);
  mk_layer_destroy(nullptr);
  CHECK(mk_model_state_bytes(0, 100, 0, &b) == MK_ERR_INVALID_ARG);
  mk_model* M = nullptr;
  CHECK(mk_model_init(nullptr, 1, nullptr, nullptr, nullptr, 128, nullptr, 16, nullptr, nullptr, &M) != MK_OK);
  CHECK(mk_model_set_length(nullptr, 0) == MK_ERR_INVALID_ARG);
  CHECK(mk_model_length_ptr(nullptr) == nullptr);
  CHECK(mk_model_step(nullptr, nullptr, 1, nullptr, nullptr, nullptr, nullptr, nullptr) == MK_ERR_INVALID_ARG);
  CHECK(mk_model_sync_status(nullptr) == MK_ERR_INVALID_ARG);
  CHECK(mk_model_reset(nullptr) == MK_ERR_INVALID_ARG);
  CHECK(mk_model_set_hidden_record(nullptr, nullptr) == MK_ERR_INVALID_ARG);
  mk_model_destroy(nullptr);
  std::printf(g_fail ? "FAILED %d\n" : "C ABI host paths: all calls clean\n", g_fail);
  return g_fail ? 1 : 0;
}
