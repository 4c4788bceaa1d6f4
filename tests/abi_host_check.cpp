// Host-only check of the C ABI's validation and argument marshalling (fa2_api.cpp), built with
// g++ under AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_abi_sanitize_cpu.py.
// The kernel launchers are replaced by stubs that record the argument block they receive, so
// no GPU code is built or run: every entry point is called with invalid arguments (the status
// must come back before any launch) and with valid ones (the stub must see the sizes, pointers,
// scale form, workspace partition and dropout parameters the header documents).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa2.h"
#include "fa2_launch.hpp"

namespace {
int g_launches = 0;
fa2::FwdArgs g_fwd;
fa2::BwdArgs g_bwd;
size_t g_noalloc_part = 0;
alignas(256) unsigned char g_fake_scratch[4096];
}  // namespace

namespace fa2 {
hipError_t launch_fwd(const FwdArgs& a) {
  ++g_launches;
  g_fwd = a;
  return hipSuccess;
}
hipError_t launch_bwd(const BwdArgs& a) {
  ++g_launches;
  g_bwd = a;
  return hipSuccess;
}
hipError_t launch_bwd_pre(const BwdArgs& a) { return launch_bwd(a); }
hipError_t launch_bwd_dkdv(const BwdArgs& a) { return launch_bwd(a); }
hipError_t launch_bwd_dq(const BwdArgs& a) { return launch_bwd(a); }
hipError_t launch_bwd_noalloc(BwdArgs a, size_t part_bytes) {
  g_noalloc_part = part_bytes;
  a.delta = reinterpret_cast<float*>(g_fake_scratch);
  a.lse2 = reinterpret_cast<float*>(g_fake_scratch + part_bytes);
  return launch_bwd(a);
}
}  // namespace fa2

static int g_fail = 0;
#define CHECK(cond)                                                    \
  do {                                                                 \
    if (!(cond)) {                                                     \
      std::fprintf(stderr, "%s:%d: CHECK(%s)\n", __FILE__, __LINE__, #cond); \
      ++g_fail;                                                        \
    }                                                                  \
  } while (0)

int main() {
  // Fake, aligned, never dereferenced device addresses (the stubs never touch them).
  void* const P = reinterpret_cast<void*>(uintptr_t(0x10000));
  float* const F = reinterpret_cast<float*>(uintptr_t(0x20000));
  void* const MIS = reinterpret_cast<void*>(uintptr_t(0x10004));
  const float sc = 0.125f;

  // ---- forward: invalid arguments return before any launch
  int before = g_launches;
  CHECK(fa2_fwd(nullptr, P, P, P, F, 1, 1, 16, 64, 0, sc, nullptr) == FA2_ERR_INVALID_ARGUMENT);
  CHECK(fa2_fwd(P, P, P, P, reinterpret_cast<float*>(MIS), 1, 1, 16, 64, 0, sc, nullptr) ==
        FA2_ERR_INVALID_ARGUMENT);
  CHECK(fa2_fwd(P, P, P, P, F, -1, 1, 16, 64, 0, sc, nullptr) == FA2_ERR_INVALID_ARGUMENT);
  CHECK(fa2_fwd(P, P, P, P, F, 1, 1, 16, 96, 0, sc, nullptr) == FA2_ERR_UNSUPPORTED);
  CHECK(fa2_fwd(P, P, P, P, F, 1, 1, 16, 64, 0, NAN, nullptr) == FA2_ERR_INVALID_ARGUMENT);
  CHECK(fa2_fwd(P, P, P, P, F, 1, 1, 16, 64, 0, 3e38f, nullptr) == FA2_ERR_INVALID_ARGUMENT);
  CHECK(fa2_fwd(P, P, P, P, F, 1 << 20, 1 << 10, 1 << 20, 128, 0, sc, nullptr) ==
        FA2_ERR_INVALID_ARGUMENT);
  CHECK(fa2_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 3, 16, 64, 1, sc, nullptr) ==
        FA2_OK);  // empty
  CHECK(fa2_fwd_gqa(P, P, P, P, F, 2, 8, 3, 16, 64, 3 * 16 * 64, 0, sc, nullptr) ==
        FA2_ERR_INVALID_ARGUMENT);  // Hkv does not divide H
  CHECK(fa2_fwd_gqa(P, P, P, P, F, 2, 8, 2, 16, 64, 2 * 16 * 64 - 8, 0, sc, nullptr) ==
        FA2_ERR_INVALID_ARGUMENT);  // K/V batch stride too small
  CHECK(fa2_fwd_dropout(P, P, P, P, F, 1, 2, 2, 16, 64, 2 * 16 * 64, 0, sc, 1.0f, 1, 2,
                        nullptr) == FA2_ERR_INVALID_ARGUMENT);  // p = 1
  CHECK(g_launches == before);

  // ---- forward: valid calls reach the launcher with the documented argument block
  CHECK(fa2_fwd(P, P, P, P, F, 2, 3, 100, 128, 1, sc, nullptr) == FA2_OK);
  CHECK(g_launches == before + 1);
  CHECK(g_fwd.B == 2 && g_fwd.H == 3 && g_fwd.Hkv == 3 && g_fwd.N == 100 && g_fwd.d == 128);
  CHECK(g_fwd.causal && !g_fwd.dropout && g_fwd.kv_bstride == 3LL * 100 * 128);
  CHECK(g_fwd.q_and == ~0u && g_fwd.q_xor == 0u);
  CHECK(std::fabs(g_fwd.scale_log2 - sc * 1.4426950408889634f) < 1e-7f);
  CHECK(fa2_fwd(P, P, P, P, F, 1, 1, 16, 64, 0, -0.5f, nullptr) == FA2_OK);
  CHECK(g_fwd.q_and == ~0u && g_fwd.q_xor == 0x80008000u);
  CHECK(std::fabs(g_fwd.scale_log2 - 0.5f * 1.4426950408889634f) < 1e-7f);
  CHECK(fa2_fwd(P, P, P, P, F, 1, 1, 16, 64, 0, 0.0f, nullptr) == FA2_OK);
  CHECK(g_fwd.q_and == 0u && g_fwd.q_xor == 0u && g_fwd.scale_log2 > 0.f);
  CHECK(fa2_fwd_dropout(P, P, P, P, F, 1, 4, 2, 16, 64, 2 * 2 * 16 * 64, 0, sc, 0.25f,
                        0x123456789ull, 7, nullptr) == FA2_OK);
  CHECK(g_fwd.dropout && g_fwd.Hkv == 2 && g_fwd.kv_bstride == 2LL * 2 * 16 * 64);
  CHECK(g_fwd.drop_thr == (16384u << 16) && g_fwd.drop_scale == 4.0f / 3.0f);
  CHECK(fa2_fwd_dropout(P, P, P, P, F, 1, 4, 2, 16, 64, 2 * 16 * 64, 0, sc, 0.0f, 1, 2,
                        nullptr) == FA2_OK);
  CHECK(!g_fwd.dropout);

  // ---- backward: workspace size and partition
  const size_t ws = fa2_bwd_workspace_bytes(2, 3, 100, 64);
  CHECK(ws == 2 * 2560);  // two parts of 2*3*100 floats, each rounded up to 256 bytes
  CHECK(fa2_bwd_workspace_bytes(0, 3, 100, 64) == 0 && fa2_bwd_workspace_bytes(1, 1, 8, 80) == 0);
  alignas(256) static unsigned char wsbuf[4 << 20];
  before = g_launches;
  CHECK(fa2_bwd(P, P, P, P, P, F, P, P, P, wsbuf, ws - 1, 2, 3, 100, 64, 1, sc, nullptr) ==
        FA2_ERR_INVALID_ARGUMENT);
  CHECK(fa2_bwd(P, P, P, P, P, F, P, nullptr, P, wsbuf, ws, 2, 3, 100, 64, 1, sc, nullptr) ==
        FA2_ERR_INVALID_ARGUMENT);
  CHECK(fa2_bwd(P, P, P, P, P, F, P, P, P, wsbuf + 8, ws, 2, 3, 100, 64, 1, sc, nullptr) ==
        FA2_ERR_INVALID_ARGUMENT);
  CHECK(fa2_bwd_dq(P, P, P, P, P, F, wsbuf, ws, P, 2, 3, 100, 64, 1, INFINITY, nullptr) ==
        FA2_ERR_INVALID_ARGUMENT);
  CHECK(g_launches == before);
  CHECK(fa2_bwd(P, P, P, P, P, F, P, P, P, wsbuf, ws, 2, 3, 100, 64, 1, -sc, nullptr) == FA2_OK);
  CHECK(g_launches == before + 1);
  CHECK(reinterpret_cast<unsigned char*>(g_bwd.delta) == wsbuf);
  CHECK(reinterpret_cast<unsigned char*>(g_bwd.lse2) == wsbuf + ws / 2);
  CHECK(g_bwd.kv_split == 1 && g_bwd.kv_part == nullptr);  // minimum workspace: no split
  CHECK(g_bwd.scale == -sc && g_bwd.sgn_xor == 0x80008000u && g_bwd.sgn_and == ~0u);
  // the larger workspace lets a small problem split its dK/dV work
  const size_t ws_split = fa2_bwd_gqa_workspace_bytes(2, 3, 3, 100, 64);
  CHECK(ws_split > ws && ws_split <= sizeof(wsbuf));
  CHECK(fa2_bwd(P, P, P, P, P, F, P, P, P, wsbuf, ws_split, 2, 3, 100, 64, 1, sc, nullptr) ==
        FA2_OK);
  CHECK(g_bwd.kv_split > 1 && reinterpret_cast<unsigned char*>(g_bwd.kv_part) == wsbuf + ws);
  // the split targets 1024 workgroups under the causal mask and 512 without: 200 (key block,
  // head) pairs split into 6 and 3 parts; the workspace is sized for the causal split
  const size_t ws200 = fa2_bwd_gqa_workspace_bytes(1, 200, 200, 1, 64);
  CHECK(ws200 == 2 * 1024 + (size_t)2 * 6 * 200 * 64 * 4 && ws200 <= sizeof(wsbuf));
  CHECK(fa2_bwd(P, P, P, P, P, F, P, P, P, wsbuf, ws200, 1, 200, 1, 64, 1, sc, nullptr) == FA2_OK);
  CHECK(g_bwd.kv_split == 6);
  CHECK(fa2_bwd(P, P, P, P, P, F, P, P, P, wsbuf, ws200, 1, 200, 1, 64, 0, sc, nullptr) == FA2_OK);
  CHECK(g_bwd.kv_split == 3);
  CHECK(fa2_bwd_dropout(P, P, P, P, P, F, P, P, P, wsbuf, ws, 1, 4, 2, 16, 64, 2 * 16 * 64, 0,
                        sc, 0.5f, 3, 4, nullptr) == FA2_OK);
  CHECK(g_bwd.dropout && g_bwd.Hkv == 2 && g_bwd.drop_scale == 2.0f);

  // ---- no-allocation backward: the static scratch's limit is checked before any launch
  before = g_launches;
  const size_t max_rows = fa2_bwd_noalloc_max_rows();
  CHECK(max_rows == size_t(1) << 21);
  CHECK(fa2_bwd_noalloc(P, P, P, P, P, F, P, P, P, 1, 1, (int)max_rows + 1, 64, 0, sc,
                        nullptr) == FA2_ERR_SCRATCH_LIMIT);
  CHECK(fa2_bwd_noalloc(P, P, P, P, P, F, nullptr, P, P, 1, 1, 16, 64, 0, sc, nullptr) ==
        FA2_ERR_INVALID_ARGUMENT);
  CHECK(g_launches == before);
  CHECK(fa2_bwd_noalloc(P, P, P, P, P, F, P, P, P, 2, 3, 100, 64, 1, sc, nullptr) == FA2_OK);
  CHECK(g_launches == before + 1 && g_noalloc_part == ws / 2 && g_bwd.kv_split == 1);

  // ---- causal window (heads per window of the causal workgroup order)
  CHECK(fa2::causal_window(256, 4ll * 2048 * 64, 16, 3, 4ll << 20) == 8);    // fwd B8 H32 N2048 d64
  CHECK(fa2::causal_window(64, 4ll * 4096 * 128, 16, 1, 4ll << 20) == 2);    // fwd B4 H16 N4096 d128
  CHECK(fa2::causal_window(16, 4ll * 16384 * 128, 64, 1, 4ll << 20) == 1);   // fwd B1 H16 N16384 d128
  CHECK(fa2::causal_window(64, 4ll * 2048 * 128, 8, 1, 4ll << 20) == 4);     // dQ B4 H16 N2048 d128
  CHECK(fa2::causal_window(64, 4ll * 2048 * 128, 16, 1, 4ll << 20) == 4);    // dK/dV B4 H16 N2048 d128
  CHECK(fa2::causal_window(8, 1ll << 20, 16, 1, 4ll << 20) == 1);           // one head per XCD
  CHECK(fa2::causal_window(64, 1, 16, 1, 4ll << 20) == 8);                  // tiny heads: all of them

  CHECK(fa2::causal_window(256, 4ll * 2048 * 64, 16, 3, 0) == 32);  // budget 0: all heads
  // the budgets the launchers use: 8 MiB at d = 64 (16 heads at B8 H32 N2048), all heads above
  CHECK(fa2::window_budget(64) == (8ll << 20) && fa2::window_budget(128) == 0 &&
        fa2::window_budget(256) == 0);
  CHECK(fa2::causal_window(256, 4ll * 2048 * 64, 16, 3, fa2::window_budget(64)) == 16);
  CHECK(fa2::causal_window(64, 4ll * 4096 * 128, 16, 1, fa2::window_budget(128)) == 8);

  // ---- status strings
  CHECK(std::strcmp(fa2_status_string(FA2_ERR_SCRATCH_LIMIT), "FA2_ERR_SCRATCH_LIMIT") == 0);
  CHECK(std::strcmp(fa2_status_string(static_cast<fa2_status>(99)), "FA2_UNKNOWN_STATUS") == 0);
  CHECK(fa2_last_hip_error() == 0);

  if (g_fail) {
    std::fprintf(stderr, "%d check(s) failed\n", g_fail);
    return 1;
  }
  std::printf("abi host checks ok\n");
  return 0;
}
