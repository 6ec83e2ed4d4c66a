// CPU check of the scratch-buffer bookkeeping in
// w8a8_int8_quantized_amd/csrc/workspace.h with a stand-in allocator
// (malloc, with every live block tracked).  Exit status 0 when every check
// holds; the failing check is printed otherwise.  Built and run by
// tests/test_workspace_cpu.py (also under ThreadSanitizer).
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <set>
#include <thread>
#include <vector>

#include "../w8a8_int8_quantized_amd/csrc/workspace.h"

namespace {

std::mutex g_mu;
std::set<void*> g_live;          // blocks the stand-in allocator has handed out and not freed
std::atomic<long> g_allocs{0};
std::atomic<int> g_fail{0};

struct MockBackend {
  static bool alloc(void** p, size_t bytes) {
    *p = std::malloc(bytes);
    if (!*p) return false;
    std::lock_guard<std::mutex> lk(g_mu);
    g_live.insert(*p);
    ++g_allocs;
    return true;
  }
  static void release(void* p) {
    {
      std::lock_guard<std::mutex> lk(g_mu);
      g_live.erase(p);
    }
    std::free(p);
  }
};

bool alive(void* p) {
  std::lock_guard<std::mutex> lk(g_mu);
  return g_live.count(p) != 0;
}

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      g_fail = 1;                                                       \
    }                                                                   \
  } while (0)

using Cache = w8::WorkspaceCache<MockBackend>;

// Two host threads share one stream's slot and keep asking for more: each
// lease's buffer must stay allocated and untouched by the other thread for
// as long as the lease is held (the lease is the call's whole enqueue), and
// every buffer ever handed out stays allocated until the cache goes away.
void two_threads_one_stream() {
  std::set<void*> handed;
  std::mutex hm;
  {
    Cache cache;
    const void* stream = reinterpret_cast<const void*>(0x1234);
    auto worker = [&](int id) {
      unsigned x = 12345u + 7919u * id;
      for (int it = 0; it < 400; ++it) {
        x = x * 1664525u + 1013904223u;
        const size_t bytes = 64 + (x >> 8) % (it * 512 + 1024);   // mostly growing
        Cache::Lease ls = cache.acquire(0, stream, 0, bytes, false);
        CHECK(ls.status() == w8::kWsOk);
        unsigned char* p = static_cast<unsigned char*>(ls.ptr());
        CHECK(p && alive(p));
        {
          std::lock_guard<std::mutex> lk(hm);
          handed.insert(p);
        }
        std::memset(p, id + 1, bytes);          // "enqueue": this call's kernels use the buffer
        std::this_thread::yield();
        for (size_t i = 0; i < bytes; i += 61) CHECK(p[i] == (unsigned char)(id + 1));
      }
    };
    std::thread a(worker, 0), b(worker, 1);
    a.join();
    b.join();
    for (void* p : handed) CHECK(alive(p));     // nothing handed out was freed
    CHECK(cache.live_count() == 1);
    CHECK(cache.retired_count() + 1 >= handed.size());
  }
  for (void* p : handed) CHECK(!alive(p));      // released with the cache
}

// Growth rounds up to powers of two and retires, never frees, the old buffer.
void growth_retires() {
  Cache cache;
  const void* s = reinterpret_cast<const void*>(0x10);
  void* p1;
  {
    Cache::Lease l = cache.acquire(0, s, 0, 1000, false);
    p1 = l.ptr();
  }
  {
    Cache::Lease l = cache.acquire(0, s, 0, 1024, false);   // rounded size 1024 serves it
    CHECK(l.ptr() == p1);
  }
  void* p2;
  {
    Cache::Lease l = cache.acquire(0, s, 0, 1025, false);
    p2 = l.ptr();
    CHECK(p2 != p1);
  }
  CHECK(alive(p1) && alive(p2));
  CHECK(cache.retired_count() == 1 && cache.live_count() == 1);
  {
    Cache::Lease l = cache.acquire(0, s, 0, 100, false);    // a smaller request keeps the big buffer
    CHECK(l.ptr() == p2);
  }
}

// During a capture an existing large-enough buffer is served; anything that
// would allocate fails with kWsCapturing and allocates nothing.
void capture_rule() {
  Cache cache;
  const void* s = reinterpret_cast<const void*>(0x20);
  const long before = g_allocs;
  {
    Cache::Lease l = cache.acquire(0, s, 0, 4096, true);
    CHECK(l.status() == w8::kWsCapturing && l.ptr() == nullptr);
  }
  CHECK(g_allocs == before);
  void* p;
  {
    Cache::Lease l = cache.acquire(0, s, 0, 4096, false);
    p = l.ptr();
  }
  {
    Cache::Lease l = cache.acquire(0, s, 0, 2048, true);
    CHECK(l.status() == w8::kWsOk && l.ptr() == p);
  }
  {
    Cache::Lease l = cache.acquire(0, s, 0, 8192, true);
    CHECK(l.status() == w8::kWsCapturing && l.ptr() == nullptr);
  }
  CHECK(g_allocs == before + 1);
  {
    // a call that needs no scratch neither allocates nor fails during a capture
    Cache::Lease l = cache.acquire(0, reinterpret_cast<const void*>(0x21), 0, 0, true);
    CHECK(l.status() == w8::kWsOk && l.ptr() == nullptr);
  }
  CHECK(g_allocs == before + 1);
}

// Streams, slots and devices get separate buffers; a call holding slot 1 may
// take slot 0 (recursive lock); another thread waits for both to be released.
void keys_and_nesting() {
  Cache cache;
  const void* s1 = reinterpret_cast<const void*>(0x30);
  const void* s2 = reinterpret_cast<const void*>(0x31);
  std::atomic<bool> other_got{false};
  std::thread t;
  {
    Cache::Lease a = cache.acquire(0, s1, 1, 512, false);
    Cache::Lease b = cache.acquire(0, s1, 0, 512, false);   // nested, same thread
    Cache::Lease c = cache.acquire(0, s2, 0, 512, false);
    Cache::Lease d = cache.acquire(1, s1, 0, 512, false);
    CHECK(a.ptr() != b.ptr() && b.ptr() != c.ptr() && b.ptr() != d.ptr() && c.ptr() != d.ptr());
    t = std::thread([&] {
      Cache::Lease e = cache.acquire(0, s2, 0, 16, false);
      other_got = true;
    });
    std::this_thread::sleep_for(std::chrono::milliseconds(50));
    CHECK(!other_got);                           // blocked while this thread holds leases
  }                                              // leases released: the other thread proceeds
  t.join();
  CHECK(other_got);
}

}  // namespace

int main() {
  two_threads_one_stream();
  growth_retires();
  capture_rule();
  keys_and_nesting();
  if (g_fail) return 1;
  std::printf("workspace bookkeeping: all checks passed\n");
  return 0;
}
