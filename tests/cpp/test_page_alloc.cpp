// Host unit test of the paged store's page allocator (built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_host_cpu.py).
#include <cstdio>
#include <cstdlib>
#include <set>
#include <vector>

#include "page_alloc.hpp"

#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "CHECK failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                    \
    }                                                              \
  } while (0)

int main() {
  lora::PageAllocator a(100);
  CHECK(a.free_count() == 100);
  std::vector<int32_t> p1, p2, p3, bad;
  CHECK(a.allocate(30, p1));
  for (int i = 0; i < 30; ++i) CHECK(p1[i] == i);          // fresh pool: ascending pages
  CHECK(a.allocate(50, p2));
  CHECK(a.free_count() == 20);
  CHECK(!a.allocate(21, p3));                              // out of pages: no side effect
  CHECK(a.free_count() == 20);
  CHECK(a.release(p1));                                    // evict the first adapter
  CHECK(a.free_count() == 50);
  CHECK(!a.release(p1));                                   // double release refused
  CHECK(a.free_count() == 50);
  CHECK(a.allocate(45, p3));                               // fragmented: reuses freed + tail pages
  std::set<int32_t> s3(p3.begin(), p3.end());
  CHECK(s3.size() == 45);
  for (int32_t q : p2) CHECK(!s3.count(q));                // no page held twice
  for (int32_t q : p3) CHECK(a.is_used(q));
  bad = {p2[0], p2[0]};
  CHECK(!a.release(bad));                                  // duplicate in one release refused
  CHECK(a.is_used(p2[0]));
  bad = {-1};
  CHECK(!a.release(bad));
  bad = {100};
  CHECK(!a.release(bad));
  CHECK(a.release(p2) && a.release(p3));
  CHECK(a.free_count() == 100);                            // conservation
  CHECK(a.allocate(0, p1) && p1.empty());
  CHECK(!a.allocate(-1, p1));
  lora::PageAllocator z(0);
  CHECK(!z.allocate(1, p1) && z.free_count() == 0);
  std::puts("page allocator: ok");
  return 0;
}
