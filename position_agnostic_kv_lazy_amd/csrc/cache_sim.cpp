// Trace-driven simulation of a document KV cache (host only).
//
// The hit-ratio argument of "LazyAttention" §2 (Eqs. 1-3, Table 1): a
// position-agnostic cache keeps one entry per document, so a budget of C
// entries holds C documents; a position-aware cache keeps one entry per
// (document, prompt position), so the same budget holds about C / D documents
// when each may appear at D positions.  This simulator replays an access trace
// against either keying under LRU eviction or a static cache of the most
// popular entries (documents are numbered by popularity rank, 0 = most
// popular), and counts hits.
#include <cstdint>
#include <list>
#include <string>
#include <unordered_map>

#include "lazy_attn.h"

namespace lazyattn {

int64_t simulate_cache(int64_t n, const int64_t* docs, const int32_t* pos, int64_t capacity,
                       int policy, int eviction, int32_t num_positions) {
  const bool aware = policy == LA_CACHE_POSITION_AWARE;
  auto key_of = [&](int64_t i) -> uint64_t {
    return aware ? (static_cast<uint64_t>(docs[i]) * static_cast<uint64_t>(num_positions) +
                    static_cast<uint64_t>(pos[i]))
                 : static_cast<uint64_t>(docs[i]);
  };
  int64_t hits = 0;
  if (eviction == LA_EVICT_STATIC_TOP) {
    // agnostic: documents 0 .. C-1; aware: all D copies of documents 0 .. C/D - 1
    const int64_t top = aware ? capacity / num_positions : capacity;
    for (int64_t i = 0; i < n; ++i) hits += docs[i] < top ? 1 : 0;
    return hits;
  }
  if (capacity == 0) return 0;
  std::list<uint64_t> order;  // front = most recently used
  std::unordered_map<uint64_t, std::list<uint64_t>::iterator> where;
  where.reserve(static_cast<size_t>(capacity) * 2);
  for (int64_t i = 0; i < n; ++i) {
    const uint64_t k = key_of(i);
    auto it = where.find(k);
    if (it != where.end()) {
      ++hits;
      order.splice(order.begin(), order, it->second);
      continue;
    }
    if (static_cast<int64_t>(order.size()) == capacity) {
      where.erase(order.back());
      order.pop_back();
    }
    order.push_front(k);
    where[k] = order.begin();
  }
  return hits;
}

}  // namespace lazyattn
