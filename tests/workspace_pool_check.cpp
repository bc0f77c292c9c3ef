// Host-only check of the workspace registry's retire logic (built with g++
// by tests/test_workspace_pool.py; no HIP).  A fake allocator hands out
// distinct addresses and records them; nothing may be freed.
#include <stdio.h>
#include <stdlib.h>

#include <set>

#include "../block_scaled_mxfp4_bf16_amd/csrc/workspace_pool.hpp"

static std::set<void *> g_alloced;
static size_t g_next = 0x10000;
static bool g_fail = false;

static int fake_alloc(int, void *, size_t bytes, void **out) {
  if (g_fail) return 4;
  *out = (void *)g_next;
  g_next += (bytes + 4095) & ~(size_t)4095;
  g_alloced.insert(*out);
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
  printf("workspace pool ok\n");
  return 0;
}
