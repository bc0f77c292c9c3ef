// Registry of library-owned workspaces, one per (device, stream).
//
// A buffer that has been handed out is never freed while the process runs:
// a HIP graph captured earlier keeps its address, and replaying the graph
// writes tickets and partial sums there.  When a call needs more than the
// current buffer holds, a larger one replaces it for later calls and the old
// one is retired -- kept allocated -- so earlier graphs stay valid.  Growth
// at least doubles the size, so the memory retired over a process's life is
// at most about the size of the live buffer.
//
// Free of HIP types: the allocator is passed in (the library binds it to
// hipMalloc plus a zero-fill launch), so the bookkeeping can be exercised on
// the host alone.
#pragma once

#include <stddef.h>

#include <mutex>
#include <vector>

namespace mxfp4 {

template <class Alloc>
class WorkspacePool {
 public:
  explicit WorkspacePool(Alloc alloc) : alloc_(alloc) {}

  // Buffer of at least `need` bytes (rounded up to 256) for (device,
  // stream); *out is null for need == 0.  Returns the allocator's status
  // (0 for success); on failure the registry is unchanged.
  int get(int device, void *stream, size_t need, void **out) {
    *out = nullptr;
    if (need == 0) return 0;
    need = (need + 255) & ~(size_t)255;
    std::lock_guard<std::mutex> lk(mu_);
    for (Entry &e : live_) {
      if (e.device != device || e.stream != stream) continue;
      if (e.bytes >= need) {
        *out = e.ptr;
        return 0;
      }
      size_t bytes = e.bytes * 2 > need ? e.bytes * 2 : need;
      void *p = nullptr;
      if (int st = alloc_(device, stream, bytes, &p)) return st;
      retired_.push_back(e);
      e.ptr = p;
      e.bytes = bytes;
      *out = p;
      return 0;
    }
    void *p = nullptr;
    if (int st = alloc_(device, stream, need, &p)) return st;
    live_.push_back(Entry{device, stream, p, need});
    *out = p;
    return 0;
  }

  // Bytes held, live and retired (for tests).
  size_t live_bytes() const {
    std::lock_guard<std::mutex> lk(mu_);
    size_t n = 0;
    for (const Entry &e : live_) n += e.bytes;
    return n;
  }
  size_t retired_bytes() const {
    std::lock_guard<std::mutex> lk(mu_);
    size_t n = 0;
    for (const Entry &e : retired_) n += e.bytes;
    return n;
  }
  size_t retired_count() const {
    std::lock_guard<std::mutex> lk(mu_);
    return retired_.size();
  }

 private:
  struct Entry {
    int device;
    void *stream;
    void *ptr;
    size_t bytes;
  };
  Alloc alloc_;
  mutable std::mutex mu_;
  std::vector<Entry> live_;
  std::vector<Entry> retired_;  // still allocated: earlier graphs may use them
};

}  // namespace mxfp4
