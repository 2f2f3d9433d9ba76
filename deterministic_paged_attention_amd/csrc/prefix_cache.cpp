// Host-side prefix cache of KV pages (see prefix_cache.h for the rules).
#include "prefix_cache.h"

#include <algorithm>

namespace bi {

namespace {
constexpr uint64_t kRollBase = 0x100000001b3ULL;     // odd multiplier of the polynomial hash
constexpr uint64_t kRollSeed = 0xcbf29ce484222325ULL;
}  // namespace

PrefixCache::PrefixCache(int32_t num_pages, int32_t page_size, int32_t hash_bits)
    : page_size_(page_size), hash_bits_(std::min(std::max(hash_bits, 0), 64)), pages_(num_pages) {
  free_.reserve(num_pages);
  // Popped from the back: pages are handed out in increasing id order.
  for (int32_t p = num_pages - 1; p >= 0; --p) free_.push_back(p);
}

// Polynomial rolling hash over the token prefix, continued page by page:
// H(prefix + page) = (...(H(prefix) * B + t0 + 1) * B + t1 + 1 ...) mod 2^64.
uint64_t PrefixCache::roll(uint64_t h, const int32_t* tokens) const {
  for (int32_t i = 0; i < page_size_; ++i) h = h * kRollBase + (uint64_t)(uint32_t)tokens[i] + 1;
  return h;
}

void PrefixCache::touch(int32_t p) { pages_[p].tick = ++clock_; }

void PrefixCache::make_evictable_if_leaf(int32_t p) {
  const Page& pg = pages_[p];
  if (pg.registered && pg.ref == 0 && pg.children == 0) evictable_.insert({pg.tick, p});
}

int32_t PrefixCache::match(const int32_t* tokens, int64_t num_tokens, int32_t* pages_out, int32_t max_pages) {
  int32_t k = 0;
  int32_t parent = -1;
  uint64_t h = kRollSeed;
  while (k < max_pages && (int64_t)(k + 1) * page_size_ <= num_tokens) {
    const int32_t* tk = tokens + (int64_t)k * page_size_;
    h = roll(h, tk);
    int32_t found = -1;
    auto range = index_.equal_range(key(h));
    for (auto it = range.first; it != range.second; ++it) {
      const Page& c = pages_[it->second];
      // The hash only nominates; reuse needs the exact tokens, depth and parent.
      if (c.registered && c.depth == k && c.parent == parent &&
          std::equal(c.tokens.begin(), c.tokens.end(), tk)) {
        found = it->second;
        break;
      }
    }
    if (found < 0) break;
    pages_out[k++] = found;
    parent = found;
  }
  for (int32_t i = 0; i < k; ++i) {
    Page& pg = pages_[pages_out[i]];
    if (pg.ref == 0) evictable_.erase({pg.tick, pages_out[i]});
    ++pg.ref;
    touch(pages_out[i]);
  }
  return k;
}

void PrefixCache::evict(int32_t p) {
  Page& pg = pages_[p];
  evictable_.erase({pg.tick, p});
  auto range = index_.equal_range(key(pg.hash));
  for (auto it = range.first; it != range.second; ++it)
    if (it->second == p) {
      index_.erase(it);
      break;
    }
  const int32_t parent = pg.parent;
  pg = Page();
  free_.push_back(p);
  ++evictions_;
  if (parent >= 0) {
    --pages_[parent].children;
    make_evictable_if_leaf(parent);
  }
}

bool PrefixCache::alloc(int32_t n, int32_t* pages_out) {
  if (n < 0) return false;
  // Evicting a leaf can expose its parent as a new leaf, so the number of
  // pages eviction can free is every registered page without a reference
  // in its subtree; count them before changing anything.
  if ((int64_t)free_.size() < n) {
    int64_t reclaimable = 0;
    std::vector<int32_t> blocked(pages_.size(), 0);  // a referenced page blocks itself and its ancestors
    for (int32_t p = 0; p < (int32_t)pages_.size(); ++p)
      if (pages_[p].registered && pages_[p].ref > 0)
        for (int32_t q = p; q >= 0 && !blocked[q]; q = pages_[q].parent) blocked[q] = 1;
    for (int32_t p = 0; p < (int32_t)pages_.size(); ++p)
      if (pages_[p].registered && !blocked[p]) ++reclaimable;
    if ((int64_t)free_.size() + reclaimable < n) return false;
  }
  for (int32_t i = 0; i < n; ++i) {
    if (free_.empty()) evict(evictable_.begin()->second);  // least recently used leaf
    const int32_t p = free_.back();
    free_.pop_back();
    Page& pg = pages_[p];
    pg = Page();
    pg.ref = 1;
    touch(p);
    pages_out[i] = p;
  }
  return true;
}

int PrefixCache::register_page(int32_t page, int32_t parent, int32_t depth, const int32_t* tokens,
                               int32_t* existing) {
  *existing = -1;
  Page& pg = pages_[page];
  if (pg.registered || pg.ref != 1) return -1;
  if (depth < 0 || (depth == 0) != (parent < 0)) return -2;
  if (parent >= 0 && (!pages_[parent].registered || pages_[parent].depth != depth - 1)) return -2;
  const uint64_t h = roll(parent >= 0 ? pages_[parent].hash : kRollSeed, tokens);
  auto range = index_.equal_range(key(h));
  for (auto it = range.first; it != range.second; ++it) {
    const Page& c = pages_[it->second];
    if (c.depth == depth && c.parent == parent && std::equal(c.tokens.begin(), c.tokens.end(), tokens)) {
      *existing = it->second;
      return 1;
    }
  }
  pg.registered = true;
  pg.parent = parent;
  pg.depth = depth;
  pg.hash = h;
  pg.tokens.assign(tokens, tokens + page_size_);
  if (parent >= 0) {
    Page& par = pages_[parent];
    if (par.children == 0 && par.ref == 0) evictable_.erase({par.tick, parent});
    ++par.children;
  }
  index_.insert({key(h), page});
  touch(page);
  return 0;
}

bool PrefixCache::release(const int32_t* pages, int32_t n) {
  std::vector<int32_t> drops(pages_.size(), 0);
  for (int32_t i = 0; i < n; ++i) {
    if (pages[i] < 0) continue;
    if (pages[i] >= (int32_t)pages_.size()) return false;
    if (++drops[pages[i]] > pages_[pages[i]].ref) return false;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t p = pages[i];
    if (p < 0) continue;
    Page& pg = pages_[p];
    --pg.ref;
    if (pg.ref > 0) continue;
    if (pg.registered) {
      make_evictable_if_leaf(p);
    } else {
      pg = Page();
      free_.push_back(p);
    }
  }
  return true;
}

bool PrefixCache::writable(int32_t page) const {
  const Page& pg = pages_[page];
  return !pg.registered && pg.ref == 1;
}

void PrefixCache::stats(int64_t out[4]) const {
  int64_t reg = 0;
  for (const Page& pg : pages_) reg += pg.registered ? 1 : 0;
  out[0] = (int64_t)free_.size();
  out[1] = reg;
  out[2] = (int64_t)evictable_.size();
  out[3] = evictions_;
}

}  // namespace bi
