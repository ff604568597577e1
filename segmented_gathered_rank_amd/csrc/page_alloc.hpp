// Host-side page allocator of the paged adapter store (pure C++, no HIP).
//
// The store is an array of fixed-size pages ("Thousands of adapters",
// slide 8: a page holds H elements; a rank-R adapter takes R pages).  Pages
// are handed out one by one, so an adapter's pages need not be contiguous and
// adapters of different ranks never fragment the pool: any free page fits any
// request.  Free pages are kept on a stack; a fresh pool hands out pages in
// ascending order, and pages returned by an eviction are reused first.
#pragma once

#include <cstdint>
#include <vector>

namespace lora {

class PageAllocator {
 public:
  explicit PageAllocator(int64_t n_pages = 0) { reset(n_pages); }

  void reset(int64_t n_pages) {
    n_pages_ = n_pages;
    free_.clear();
    free_.reserve(static_cast<size_t>(n_pages));
    for (int64_t p = n_pages - 1; p >= 0; --p) free_.push_back(static_cast<int32_t>(p));
    used_.assign(static_cast<size_t>(n_pages), 0);
  }

  int64_t n_pages() const { return n_pages_; }
  int64_t free_count() const { return static_cast<int64_t>(free_.size()); }

  // Takes `count` pages.  On failure returns false and changes nothing.
  bool allocate(int64_t count, std::vector<int32_t>& out) {
    if (count < 0 || count > free_count()) return false;
    out.clear();
    out.reserve(static_cast<size_t>(count));
    for (int64_t i = 0; i < count; ++i) {
      int32_t p = free_.back();
      free_.pop_back();
      used_[static_cast<size_t>(p)] = 1;
      out.push_back(p);
    }
    return true;
  }

  // Returns pages.  Refuses (returns false, changes nothing) if any page is out
  // of range, not held, or listed twice.
  bool release(const std::vector<int32_t>& pages) {
    std::vector<uint8_t> seen;
    for (int32_t p : pages) {
      if (p < 0 || p >= n_pages_ || !used_[static_cast<size_t>(p)]) return false;
    }
    seen.assign(static_cast<size_t>(n_pages_), 0);
    for (int32_t p : pages) {
      if (seen[static_cast<size_t>(p)]) return false;
      seen[static_cast<size_t>(p)] = 1;
    }
    for (auto it = pages.rbegin(); it != pages.rend(); ++it) {
      used_[static_cast<size_t>(*it)] = 0;
      free_.push_back(*it);
    }
    return true;
  }

  bool is_used(int32_t p) const {
    return p >= 0 && p < n_pages_ && used_[static_cast<size_t>(p)];
  }

 private:
  int64_t n_pages_ = 0;
  std::vector<int32_t> free_;
  std::vector<uint8_t> used_;
};

}  // namespace lora
