// Host unit test of the launch-size guard (built with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_host_cpu.py).
#include <cstdint>
#include <cstdio>

#include "launch_limits.hpp"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "CHECK failed line %d: %s\n", __LINE__, #c); \
      return 1;                                                         \
    }                                                                   \
  } while (0)

int main() {
  using lora::grid_fits;
  const int64_t max_items = 4294967295LL;   // 2^32 - 1 work-items
  CHECK(grid_fits(1, 256));
  CHECK(grid_fits(max_items / 256, 256));          // 16,777,215 workgroups of 256
  CHECK(!grid_fits(max_items / 256 + 1, 256));     // one more workgroup overflows the grid
  CHECK(!grid_fits(INT32_MAX, 256));               // the old guard's bound, far beyond the grid
  CHECK(grid_fits(max_items, 1));
  CHECK(!grid_fits(max_items + 1, 1));
  CHECK(grid_fits(max_items / 512, 512));
  CHECK(!grid_fits(0, 256));
  CHECK(!grid_fits(-5, 256));
  CHECK(!grid_fits(10, 0));
  CHECK(!grid_fits(INT64_MAX, 1024));              // no overflow in the check itself
  std::puts("launch limits ok");
  return 0;
}
