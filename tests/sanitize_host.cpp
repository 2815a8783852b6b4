// Randomised calls of every host-side function of the C ABI (the planner, the
// size queries, the entry points' validation and logging), for a build of the
// library's host code with the compiler's address and undefined-behaviour
// checks (tests/test_sanitize_host.py builds and runs it).  The build holds no
// device code, so an entry-point call that passes validation fails at its
// launch: the fake addresses below are never read and nothing runs.
// Prints "OK <calls>" and exits 0 unless a check stops it first.
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "conv1d_gn.h"

namespace {

uint64_t rng = 0x9e3779b97f4a7c15ull;
uint64_t next() {  // xorshift64*
  rng ^= rng >> 12;
  rng ^= rng << 25;
  rng ^= rng >> 27;
  return rng * 0x2545f4914f6cdd1dull;
}

const int64_t kEdges64[] = {-1,           0,           1,           2,           65535,
                            65536,        1ll << 30,   (1ll << 30) + 1, 1ll << 31, 1ll << 32,
                            1ll << 40,    (1ll << 40) + 1, 1ll << 46, 1ll << 62,
                            (1ll << 62) + 1, INT64_MAX, INT64_MIN};
const int32_t kEdges32[] = {-1, 0, 1, 2, 3, 5, 8, 9, 16, 1 << 15, 1 << 30, INT32_MAX, INT32_MIN};

// small plausible values most of the time, else an edge or any value of the type
int64_t pick64(int64_t lo, int64_t hi) {
  const uint64_t r = next() % 8;
  if (r < 6) return lo + (int64_t)(next() % (uint64_t)(hi - lo + 1));
  if (r == 6) return kEdges64[next() % (sizeof(kEdges64) / sizeof(kEdges64[0]))];
  return (int64_t)next();
}
int32_t pick32(int32_t lo, int32_t hi) {
  const uint64_t r = next() % 8;
  if (r < 6) return lo + (int32_t)(next() % (uint64_t)(hi - lo + 1));
  if (r == 6) return kEdges32[next() % (sizeof(kEdges32) / sizeof(kEdges32[0]))];
  return (int32_t)next();
}
float pick_eps() {
  switch (next() % 8) {
    case 0: return 0.f;
    case 1: return -1e-5f;
    case 2: return 1.f / 0.f;
    case 3: return 0.f / 0.f;
    default: return 1e-5f;
  }
}

}  // namespace

int main(int argc, char** argv) {
  const long iters = argc > 1 ? std::atol(argv[1]) : 100000;
  void* f = (void*)(uintptr_t)(1u << 20);
  const float* ff = (const float*)f;
  long calls = 0;
  for (long i = 0; i < iters; ++i) {
    // the log's formatting and the route override take part now and then
    if (i % 997 == 0) setenv("C1G_LOG", "1", 1);
    if (i % 997 == 50) unsetenv("C1G_LOG");
    if (i % 13 == 0) setenv("C1G_FORCE_PATH", "split", 1);
    if (i % 13 == 1) unsetenv("C1G_FORCE_PATH");
    c1g_conv_desc d;
    d.N = pick64(0, 70);
    d.C_in = pick64(1, 600);
    d.C_out = pick64(1, 600);
    d.T = next() % 4 == 0 ? 1 : pick64(1, 5000);
    d.K = pick32(1, 10);
    d.stride = pick32(1, 4);
    d.dilation = pick32(1, 4);
    d.pad_left = pick32(0, 10);
    d.pad_right = pick32(0, 10);
    d.dtype = pick32(0, 1);
    d.out_dtype = pick32(0, 1);
    d.x_layout = pick32(0, 1);
    c1g_norm_desc nd;
    nd.norm = pick32(0, 2);
    nd.G = pick32(1, 64);
    nd.eps = pick_eps();
    nd.epilogue = pick32(0, 1);
    nd.flags = pick32(0, 7);
    const size_t ws = (size_t)next() >> (next() % 64);

    (void)c1g_out_len(&d);
    (void)c1g_check(&d, &nd, ws);
    (void)c1g_check(&d, nullptr, ws);
    (void)c1g_route(&d, &nd);
    (void)c1g_route(&d, nullptr);
    (void)c1g_conv1d_workspace_size(&d);
    (void)c1g_conv1d_gn_workspace_size(&d, &nd);
    (void)conv1d_forward(&d, f, f, ff, f, f, ws, nullptr);
    (void)conv1d_gn_forward(&d, &nd, f, f, ff, ff, ff, ff, f, nullptr, nullptr, f, ws, nullptr);
    (void)conv1d_gn_forward_noalloc(&d, &nd, f, f, ff, ff, ff, ff, f, nullptr, nullptr, nullptr);
    const int64_t N = pick64(0, 64), C = pick64(1, 512), L = pick64(1, 5000);
    const int32_t G = pick32(1, 64);
    (void)c1g_gn_stats_workspace_size(N, C, L, G);
    (void)gn_stats(N, C, L, G, pick_eps(), ff, (float*)f, (float*)f, f, ws, nullptr);
    (void)gn_apply(N, C, L, G, ff, ff, ff, nullptr, nullptr, (float*)f, nullptr);
    (void)gn_apply_bf16(N, C, L, G, (const uint16_t*)f, ff, ff, nullptr, nullptr, (uint16_t*)f,
                        nullptr);
    (void)c1g_status_string((int)(next() % 8) - 1);
    calls += 16;
  }
  // the null descriptors
  (void)c1g_out_len(nullptr);
  (void)c1g_check(nullptr, nullptr, 0);
  (void)c1g_route(nullptr, nullptr);
  (void)conv1d_forward(nullptr, f, f, ff, f, f, 0, nullptr);
  (void)conv1d_gn_forward(nullptr, nullptr, f, f, ff, ff, ff, ff, f, nullptr, nullptr, f, 0,
                          nullptr);
  std::printf("OK %ld\n", calls);
  return 0;
}
