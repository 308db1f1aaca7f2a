// Process-lifetime lookup table of the host code: results of slow runtime
// queries (occupancy, attributes) kept per (device, kernel).  It is a plain
// array behind a spin lock, trivially destructible, so the library leaves no
// destructor of its own to run when the process exits.
#pragma once

#include <atomic>
#include <type_traits>

namespace dspark {

template <typename V, int N = 64>
class KeyedCache {
 public:
  // True and the stored value when (dev, key) is present.
  bool find(int dev, const void* key, V& out) {
    Lock l(busy_);
    for (int i = 0; i < n_; ++i)
      if (e_[i].dev == dev && e_[i].key == key) {
        out = e_[i].v;
        return true;
      }
    return false;
  }
  // Store (or replace) the value of (dev, key); a full table stores nothing,
  // which only means the query is made again next time.
  void put(int dev, const void* key, const V& v) {
    Lock l(busy_);
    for (int i = 0; i < n_; ++i)
      if (e_[i].dev == dev && e_[i].key == key) {
        e_[i].v = v;
        return;
      }
    if (n_ < N) e_[n_++] = Entry{dev, key, v};
  }

 private:
  struct Entry {
    int dev;
    const void* key;
    V v;
  };
  struct Lock {
    std::atomic_flag& f;
    explicit Lock(std::atomic_flag& flag) : f(flag) {
      while (f.test_and_set(std::memory_order_acquire)) {
      }
    }
    ~Lock() { f.clear(std::memory_order_release); }
  };
  std::atomic_flag busy_ = ATOMIC_FLAG_INIT;
  Entry e_[N] = {};
  int n_ = 0;
};

static_assert(std::is_trivially_destructible<KeyedCache<int>>::value,
              "process-lifetime caches must not need a destructor at exit");

}  // namespace dspark
