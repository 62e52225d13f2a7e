// Host-side plan of an elastic cache resize: which keys survive, where they
// end up, and the recency order the device lookup continues from.  Pure C++
// (no HIP), so that it can be built and checked on its own.
//
// The pages let the GPU expert-cache budget change at run time without a
// restart or a reload of the host pool (aipolix.com FreeToken article, sixth
// paragraph).  The rule (stated at expert_cache_resize in moe.h):
//  - growing appends empty slots;
//  - shrinking evicts occupied slots in ascending recency while more than
//    the new capacity are occupied, then moves every survivor held in a slot
//    at or past the new capacity (ascending slot) into the lowest empty slot
//    below it (ascending), keeping key and recency;
//  - the clock does not change.
#pragma once

#include <algorithm>
#include <cstdint>
#include <numeric>
#include <utility>
#include <vector>

namespace moe {

struct ResizePlan {
  std::vector<int32_t> key;                       // [C2] key per slot, -1 empty
  std::vector<uint64_t> stamp;                    // [C2] recency, 0 empty
  std::vector<int32_t> order;                     // [C2] packed recency order
  std::vector<std::pair<int32_t, int32_t>> moves; // (src slot >= C2, dst slot < C2)
  std::vector<int32_t> evicted;                   // keys evicted, least recent first
};

// Recency order of a slot table as the device lookup keeps it: empty slots
// by index, then occupied slots by ascending stamp; entry = slot | (key + 1)
// << key_shift.
inline std::vector<int32_t> recency_order(const std::vector<int32_t>& key,
                                          const std::vector<uint64_t>& stamp, int key_shift) {
  std::vector<int32_t> order(key.size());
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
    return (key[a] < 0 ? 0 : stamp[a]) < (key[b] < 0 ? 0 : stamp[b]);
  });
  for (auto& o : order) o |= (key[o] + 1) << key_shift;
  return order;
}

inline ResizePlan plan_resize(const std::vector<int32_t>& key, const std::vector<uint64_t>& stamp,
                              int C2, int key_shift) {
  const int C = (int)key.size();
  ResizePlan p;
  p.key.assign(C2, -1);
  p.stamp.assign(C2, 0);
  if (C2 >= C) {
    std::copy(key.begin(), key.end(), p.key.begin());
    std::copy(stamp.begin(), stamp.end(), p.stamp.begin());
  } else {
    std::vector<int> occ;
    for (int s = 0; s < C; s++)
      if (key[s] >= 0) occ.push_back(s);
    std::sort(occ.begin(), occ.end(), [&](int a, int b) { return stamp[a] < stamp[b]; });
    const size_t drop = occ.size() > (size_t)C2 ? occ.size() - C2 : 0;
    std::vector<char> alive(C, 0);
    for (size_t i = 0; i < occ.size(); i++) {
      if (i < drop)
        p.evicted.push_back(key[occ[i]]);
      else
        alive[occ[i]] = 1;
    }
    std::vector<int> holes;
    for (int s = 0; s < C2; s++) {
      if (alive[s]) {
        p.key[s] = key[s];
        p.stamp[s] = stamp[s];
      } else {
        holes.push_back(s);
      }
    }
    size_t h = 0;  // at most C2 keys survive, so the holes suffice
    for (int s = C2; s < C; s++)
      if (alive[s]) {
        const int d = holes[h++];
        p.key[d] = key[s];
        p.stamp[d] = stamp[s];
        p.moves.emplace_back(s, d);
      }
  }
  p.order = recency_order(p.key, p.stamp, key_shift);
  return p;
}

}  // namespace moe
