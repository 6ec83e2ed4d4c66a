// Host-side bookkeeping of the library's own scratch buffers: one buffer per
// (device, stream, slot) for the split-K partial tiles (slot 0) and the
// asymmetric path (slot 1).  Plain C++ (no HIP types): the allocator is a
// template parameter, so the rules below are built and tested on the CPU
// with a stand-in allocator.
//
// Rules:
//  * A call holds the cache's lock (a Lease) from the moment it obtains its
//    buffer until it has enqueued every kernel that uses it.  Two host
//    threads that share a stream therefore enqueue their kernel sequences one
//    after the other; neither can slip a kernel between the other's split-K
//    product and its reduction.  The lock is recursive: a call that takes
//    slot 1 may take slot 0 inside it.
//  * A buffer is never freed while the process runs.  A larger request gets a
//    new buffer (the size rounded up to a power of two, so a slot retires
//    less than its final size in all) and the old one is retired, not freed:
//    kernels enqueued earlier, or a graph captured with its address, may
//    still use it.
//  * During a stream capture nothing is allocated: a request that the
//    existing buffer cannot serve fails with kWsCapturing and nothing is
//    enqueued (make one such call on the stream before capturing).
#pragma once

#include <cstddef>
#include <cstdint>
#include <mutex>
#include <utility>
#include <vector>

namespace w8 {

enum WsStatus { kWsOk = 0, kWsAllocFailed = 1, kWsCapturing = 2 };

// Backend: static bool alloc(void** p, size_t bytes) (true on success) and
// static void release(void* p) (called when the cache itself is destroyed).
template <class Backend>
class WorkspaceCache {
 public:
  class Lease {
   public:
    Lease(Lease&&) = default;
    void* ptr() const { return p_; }
    WsStatus status() const { return st_; }

   private:
    friend class WorkspaceCache;
    Lease(std::unique_lock<std::recursive_mutex>&& lk, void* p, WsStatus st) : lk_(std::move(lk)), p_(p), st_(st) {}
    std::unique_lock<std::recursive_mutex> lk_;
    void* p_;
    WsStatus st_;
  };

  WorkspaceCache() = default;
  WorkspaceCache(const WorkspaceCache&) = delete;
  WorkspaceCache& operator=(const WorkspaceCache&) = delete;
  ~WorkspaceCache() {
    for (Entry& e : live_) Backend::release(e.p);
    for (void* p : retired_) Backend::release(p);
  }

  // At least `bytes` of scratch for (dev, stream, slot); `capturing` says
  // whether `stream` is being captured into a graph.  bytes == 0 (a call that
  // needs no scratch this time) takes the lock only, with a null buffer.
  Lease acquire(int dev, const void* stream, int slot, size_t bytes, bool capturing) {
    std::unique_lock<std::recursive_mutex> lk(mu_);
    if (bytes == 0) return Lease(std::move(lk), nullptr, kWsOk);
    Entry* e = find(dev, stream, slot);
    if (e && e->bytes >= bytes) return Lease(std::move(lk), e->p, kWsOk);
    if (capturing) return Lease(std::move(lk), nullptr, kWsCapturing);
    size_t sz = 256;
    while (sz < bytes) sz <<= 1;
    void* p = nullptr;
    if (!Backend::alloc(&p, sz)) return Lease(std::move(lk), nullptr, kWsAllocFailed);
    if (e) {
      retired_.push_back(e->p);
      e->p = p;
      e->bytes = sz;
    } else {
      live_.push_back({dev, stream, slot, p, sz});
    }
    return Lease(std::move(lk), p, kWsOk);
  }

  // Bookkeeping views (tests).
  size_t live_count() {
    std::lock_guard<std::recursive_mutex> lk(mu_);
    return live_.size();
  }
  size_t retired_count() {
    std::lock_guard<std::recursive_mutex> lk(mu_);
    return retired_.size();
  }

 private:
  struct Entry {
    int dev;
    const void* stream;
    int slot;
    void* p;
    size_t bytes;
  };
  Entry* find(int dev, const void* stream, int slot) {
    for (Entry& e : live_)
      if (e.dev == dev && e.stream == stream && e.slot == slot) return &e;
    return nullptr;
  }
  std::recursive_mutex mu_;
  std::vector<Entry> live_;
  std::vector<void*> retired_;
};

}  // namespace w8
