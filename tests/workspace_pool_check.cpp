// Host-only check of the workspace registry's retire logic (built with g++
// by tests/test_workspace_pool.py; no HIP).  A fake allocator hands out
// distinct addresses and records them; nothing may be freed.
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <map>
#include <mutex>
#include <random>
#include <set>
#include <thread>
#include <vector>

#include "../block_scaled_mxfp4_bf16_amd/csrc/workspace_pool.hpp"

static std::mutex g_mu;  // the fake allocator is called from several threads
static std::set<void *> g_alloced;
static std::map<void *, size_t> g_size;
static size_t g_next = 0x10000;
static bool g_fail = false;

static int fake_alloc(int, void *, size_t bytes, void **out) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_fail) return 4;
  *out = (void *)g_next;
  g_next += (bytes + 4095) & ~(size_t)4095;
  g_alloced.insert(*out);
  g_size[*out] = bytes;
  return 0;
}

// Several threads ask for workspaces on 2 devices x 4 streams at once: every
// buffer handed out was allocated, holds the request, and the registry's
// live bytes end equal to the sum of the (device, stream) buffers.
static int concurrent_check() {
  mxfp4::WorkspacePool<int (*)(int, void *, size_t, void **)> pool(fake_alloc);
  std::atomic<int> bad{0};
  std::vector<std::thread> ts;
  for (int t = 0; t < 8; ++t) {
    ts.emplace_back([&, t] {
      std::mt19937 rng(1234 + t);
      for (int i = 0; i < 4000; ++i) {
        const int dev = rng() % 2;
        void *stream = (void *)(uintptr_t)(1 + rng() % 4);
        const size_t need = 1 + rng() % (1 << 20);
        void *p = nullptr;
        if (pool.get(dev, stream, need, &p) != 0 || p == nullptr) {
          ++bad;
          continue;
        }
        std::lock_guard<std::mutex> lk(g_mu);
        auto it = g_size.find(p);
        if (it == g_size.end() || it->second < need) ++bad;
      }
    });
  }
  for (auto &th : ts) th.join();
  if (bad.load() != 0) {
    fprintf(stderr, "concurrent check: %d bad results\n", bad.load());
    return 1;
  }
  // one live buffer per (device, stream) pair that was used: 8 pairs
  size_t live = 0;
  for (int dev = 0; dev < 2; ++dev)
    for (int s = 1; s <= 4; ++s) {
      void *p = nullptr;
      if (pool.get(dev, (void *)(uintptr_t)s, 1, &p) != 0 || p == nullptr) return 1;
      std::lock_guard<std::mutex> lk(g_mu);
      live += (g_size[p] + 255) & ~(size_t)255;
    }
  if (live != pool.live_bytes()) {
    fprintf(stderr, "concurrent check: live %zu, registry says %zu\n", live, pool.live_bytes());
    return 1;
  }
  return 0;
}

#define CHECK(c)                                              \
  do {                                                        \
    if (!(c)) {                                               \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      return 1;                                               \
    }                                                         \
  } while (0)

int main() {
  mxfp4::WorkspacePool<int (*)(int, void *, size_t, void **)> pool(fake_alloc);
  void *s1 = (void *)0x1, *s2 = (void *)0x2;
  void *p = nullptr, *q = nullptr, *r = nullptr;
  CHECK(pool.get(0, s1, 0, &p) == 0 && p == nullptr);        // nothing needed
  CHECK(pool.get(0, s1, 1000, &p) == 0 && p != nullptr);     // first buffer: 1024 bytes
  CHECK(pool.live_bytes() == 1024 && pool.retired_count() == 0);
  CHECK(pool.get(0, s1, 800, &q) == 0 && q == p);            // fits: same buffer
  // growth: a new buffer of at least twice the size; the old one is retired,
  // not freed, so a graph that captured p can still replay
  CHECK(pool.get(0, s1, 1500, &q) == 0 && q != p);
  CHECK(pool.live_bytes() == 2048 && pool.retired_bytes() == 1024 && pool.retired_count() == 1);
  CHECK(g_alloced.count(p) == 1 && g_alloced.count(q) == 1);
  CHECK(pool.get(0, s1, 100000, &r) == 0 && r != q && pool.live_bytes() == 100096);
  CHECK(pool.retired_count() == 2 && pool.retired_bytes() == 1024 + 2048);
  // another stream and another device get buffers of their own
  void *a = nullptr, *b = nullptr;
  CHECK(pool.get(0, s2, 512, &a) == 0 && a != r);
  CHECK(pool.get(1, s1, 512, &b) == 0 && b != r && b != a);
  CHECK(pool.get(0, s1, 512, &p) == 0 && p == r);
  // a failed growth leaves the registry as it was
  g_fail = true;
  void *f = (void *)0x99;
  CHECK(pool.get(0, s1, 1 << 20, &f) == 4 && f == nullptr);
  g_fail = false;
  CHECK(pool.get(0, s1, 512, &p) == 0 && p == r && pool.retired_count() == 2);
  CHECK(concurrent_check() == 0);
  printf("workspace pool ok\n");
  return 0;
}
