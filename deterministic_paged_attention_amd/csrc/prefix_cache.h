// Host-side prefix cache of KV pages: which physical pages hold the KV of
// which token prefix, who holds them, and which may be reused or evicted.
//
// Rules (Vosti deep-dive blog (深入解析 Vosti), §3.2 engineering constraints
// and §5.4 exact prefix matching; §3.2 invariants 2 and 3):
//  * a rolling hash over the token prefix only proposes candidate pages; a
//    page is reused only if its tokens, its depth in the prefix and its parent
//    page all match exactly, so a hash collision can never justify reuse;
//  * registered (shared) pages are immutable; new KV goes to private pages,
//    and a page is registered only after the writes that fill it;
//  * under memory pressure only unreferenced leaves are evicted, so a parent
//    page cannot be recycled while a retained child still names it.
// Not thread-safe: one owner (the scheduler) calls it.
#pragma once

#include <stdint.h>

#include <set>
#include <unordered_map>
#include <utility>
#include <vector>

namespace bi {

class PrefixCache {
 public:
  // hash_bits in [0, 64]: the hash keeps that many low bits (fewer bits force
  // collisions; 0 makes every page a candidate for every lookup).
  PrefixCache(int32_t num_pages, int32_t page_size, int32_t hash_bits);

  int32_t num_pages() const { return (int32_t)pages_.size(); }
  int32_t page_size() const { return page_size_; }

  // Longest run of registered pages holding tokens[0 : 16 k) exactly, k <=
  // max_pages; each matched page is acquired (reference count + 1).  Returns k.
  int32_t match(const int32_t* tokens, int64_t num_tokens, int32_t* pages_out, int32_t max_pages);

  // n private pages (reference count 1, unregistered), taking free pages
  // first, then evicting unreferenced registered leaves, least recently used
  // first.  All or nothing: false (and no change) if n cannot be met.
  bool alloc(int32_t n, int32_t* pages_out);

  // Registers `page` as the cached page of tokens[0 : page_size) at `depth`
  // below `parent` (-1 at depth 0).  Returns 0 on success; 1 if an identical
  // entry (same tokens, depth and parent) is already registered (*existing
  // names it; `page` stays private); negative on a violated precondition:
  // -1 page not privately held (reference count 1, unregistered), -2 bad
  // parent/depth (the parent must be registered, at depth - 1).
  int register_page(int32_t page, int32_t parent, int32_t depth, const int32_t* tokens, int32_t* existing);

  // Drops one reference from each page (pages with no reference: -1).  An
  // unregistered page with no reference left is free again; a registered one
  // stays cached and becomes evictable once it is also a leaf.  Returns false
  // if some page had no reference (nothing is changed then).
  bool release(const int32_t* pages, int32_t n);

  bool writable(int32_t page) const;  // privately held and unregistered
  bool registered(int32_t page) const { return pages_[page].registered; }
  int32_t refs(int32_t page) const { return pages_[page].ref; }

  // free pages, registered pages, evictable pages, evictions so far
  void stats(int64_t out[4]) const;

 private:
  struct Page {
    int32_t ref = 0;
    bool registered = false;
    int32_t parent = -1;
    int32_t depth = -1;
    int32_t children = 0;      // registered pages naming this one as parent
    uint64_t hash = 0;         // rolling hash of the whole prefix through this page
    uint64_t tick = 0;         // last use, for eviction order
    std::vector<int32_t> tokens;
  };

  uint64_t roll(uint64_t h, const int32_t* tokens) const;
  uint64_t key(uint64_t h) const { return hash_bits_ >= 64 ? h : (h & ((1ULL << hash_bits_) - 1)); }
  void touch(int32_t p);
  void make_evictable_if_leaf(int32_t p);
  void evict(int32_t p);

  int32_t page_size_;
  int32_t hash_bits_;
  uint64_t clock_ = 0;
  int64_t evictions_ = 0;
  std::vector<Page> pages_;
  std::vector<int32_t> free_;                            // popped from the back
  std::unordered_multimap<uint64_t, int32_t> index_;     // key(hash) -> registered page
  std::set<std::pair<uint64_t, int32_t>> evictable_;     // (tick, page): registered, ref 0, no children
};

}  // namespace bi
