// Slot policy of the expert pool (host only, no HIP): which device slot each
// requested expert occupies, and which experts must be copied in.
//
// Pulsar README, MoE expert-resolve list: the device hot set is a fixed pool
// with touch-count admission (an expert earns a slot only by being hotter than
// the coldest resident, so the set stays stable instead of thrashing); a
// background prefetch loads the next layer's predicted experts. Rules here:
//   * every resolve call is an epoch; each requested expert's touch count
//     grows by one per epoch that requests it;
//   * slots are FREE, RESIDENT (hot set, at most n_slots - n_transient) or
//     TRANSIENT (a requested expert that was not admitted; any non-resident
//     slot may hold one);
//   * a slot last used in the current epoch is never overwritten (the kernels
//     of that epoch may still read it);
//   * a requested expert that is not in a slot is admitted to the hot set if
//     the hot set has room, or if its touch count exceeds that of the coldest
//     evictable resident (fewest touches, then least recently used, then
//     lowest slot), which it replaces; otherwise it is loaded as TRANSIENT
//     into a free slot or the least recently used evictable transient slot;
//   * a requested expert already held as TRANSIENT is promoted the same way:
//     into free hot-set room, or by exchanging roles with the coldest
//     evictable resident when it is hotter (no copy: the resident's slot
//     becomes TRANSIENT and keeps its expert);
//   * prefetch uses the same placement without touching counts, loads an
//     expert as TRANSIENT only into a free or evictable transient slot, and
//     never evicts a resident for a non-admissible expert.
#pragma once

#include <stdint.h>

#include <vector>

namespace moe {

class PoolPolicy {
 public:
  enum State : uint8_t { FREE = 0, RESIDENT = 1, TRANSIENT = 2 };
  struct Slot {
    int32_t key = -1;        // layer * n_experts + expert, -1 when free
    State state = FREE;
    int64_t last_use = -1;   // epoch of the last resolve or prefetch that placed or hit it
    bool prefetched = false; // placed by a prefetch and not yet requested
  };
  // One requested (or prefetched) expert's placement.
  struct Place {
    int32_t key;
    int32_t slot;
    bool copy;      // the expert's bytes must be copied into the slot
  };
  struct Stats {
    int64_t epochs = 0, requests = 0, hits_resident = 0, hits_transient = 0, admitted = 0,
            transient_loads = 0, promotions = 0, evictions = 0, prefetch_loads = 0,
            prefetch_hits = 0;
  };

  PoolPolicy(int n_layers, int n_experts, int n_slots, int n_transient)
      : L_(n_layers), E_(n_experts), cap_(n_slots - n_transient), slots_(n_slots),
        where_(static_cast<size_t>(n_layers) * n_experts, -1),
        touch_(static_cast<size_t>(n_layers) * n_experts, 0) {}

  // Places the experts `ids` (n entries, duplicates and ids outside [0, E)
  // ignored) of `layer` for a new epoch. Returns false, with `out` cleared,
  // when an expert finds no slot (more unique experts than the slots that
  // are not protected this epoch); the policy state is then unchanged.
  bool resolve(int layer, const int32_t* ids, int n, std::vector<Place>* out) {
    Snapshot snap = save();
    ++epoch_;
    ++st_.epochs;
    out->clear();
    std::vector<int32_t> keys = unique_keys(layer, ids, n);
    for (int32_t k : keys) ++touch_[k];
    // protect every requested expert already in a slot
    for (int32_t k : keys)
      if (where_[k] >= 0) slots_[where_[k]].last_use = epoch_;
    for (int32_t k : keys) {
      ++st_.requests;
      const int s = where_[k];
      if (s >= 0) {
        Slot& sl = slots_[s];
        if (sl.prefetched) { ++st_.prefetch_hits; sl.prefetched = false; }
        if (sl.state == RESIDENT) {
          ++st_.hits_resident;
        } else {
          ++st_.hits_transient;
          promote(s);
        }
        out->push_back({k, s, false});
        continue;
      }
      const int t = place(k);
      if (t < 0) {
        restore(snap);
        out->clear();
        return false;
      }
      out->push_back({k, t, true});
    }
    return true;
  }

  // Prefetch into the current epoch: experts not in a slot that would be
  // admitted (or fit into a free or evictable transient slot) are placed and
  // returned for copying; the others are skipped.
  void prefetch(int layer, const int32_t* ids, int n, std::vector<Place>* out) {
    out->clear();
    for (int32_t k : unique_keys(layer, ids, n)) {
      if (where_[k] >= 0) continue;
      const int t = place(k);
      if (t < 0) continue;
      slots_[t].prefetched = true;
      ++st_.prefetch_loads;
      out->push_back({k, t, true});
    }
  }

  const Stats& stats() const { return st_; }
  const std::vector<Slot>& slots() const { return slots_; }
  uint32_t touches(int32_t key) const { return touch_[key]; }
  int32_t slot_of(int32_t key) const { return where_[key]; }
  int64_t epoch() const { return epoch_; }
  int hot_capacity() const { return cap_; }

 private:
  struct Snapshot {
    std::vector<Slot> slots;
    std::vector<int32_t> where;
    std::vector<uint32_t> touch;
    int res;
    int64_t epoch;
    Stats st;
  };
  Snapshot save() const { return {slots_, where_, touch_, res_, epoch_, st_}; }
  void restore(const Snapshot& s) {
    slots_ = s.slots; where_ = s.where; touch_ = s.touch; res_ = s.res; epoch_ = s.epoch;
    st_ = s.st;
  }

  std::vector<int32_t> unique_keys(int layer, const int32_t* ids, int n) const {
    std::vector<int32_t> keys;
    if (layer < 0 || layer >= L_) return keys;
    for (int i = 0; i < n; ++i) {
      const int32_t e = ids[i];
      if (e < 0 || e >= E_) continue;
      const int32_t k = layer * E_ + e;
      bool seen = false;
      for (int32_t q : keys) seen = seen || q == k;
      if (!seen) keys.push_back(k);
    }
    return keys;
  }

  bool evictable(int s) const { return slots_[s].last_use < epoch_; }

  // coldest evictable resident: fewest touches, then oldest use, then lowest slot
  int coldest_resident() const {
    int best = -1;
    for (int s = 0; s < static_cast<int>(slots_.size()); ++s) {
      const Slot& sl = slots_[s];
      if (sl.state != RESIDENT || !evictable(s)) continue;
      if (best < 0) { best = s; continue; }
      const Slot& b = slots_[best];
      const uint32_t ts = touch_[sl.key], tb = touch_[b.key];
      if (ts < tb || (ts == tb && sl.last_use < b.last_use)) best = s;
    }
    return best;
  }
  int free_slot() const {
    for (int s = 0; s < static_cast<int>(slots_.size()); ++s)
      if (slots_[s].state == FREE) return s;
    return -1;
  }
  // least recently used evictable transient slot (lowest slot on ties)
  int lru_transient() const {
    int best = -1;
    for (int s = 0; s < static_cast<int>(slots_.size()); ++s) {
      const Slot& sl = slots_[s];
      if (sl.state != TRANSIENT || !evictable(s)) continue;
      if (best < 0 || sl.last_use < slots_[best].last_use) best = s;
    }
    return best;
  }

  void clear_slot(int s) {
    Slot& sl = slots_[s];
    if (sl.key >= 0) where_[sl.key] = -1;
    if (sl.state == RESIDENT) --res_;
    sl = Slot{};
  }
  void fill(int s, int32_t k, State st) {
    Slot& sl = slots_[s];
    sl.key = k;
    sl.state = st;
    sl.last_use = epoch_;
    sl.prefetched = false;
    where_[k] = s;
    if (st == RESIDENT) ++res_;
  }

  // A slot for key k, which is in none; -1 if there is none. Counts every
  // placement (requested or prefetched) as admitted or transient_loads.
  int place(int32_t k) {
    if (res_ < cap_) {
      int s = free_slot();
      if (s < 0) s = lru_transient();
      if (s >= 0) {
        if (slots_[s].state != FREE) ++st_.evictions;
        clear_slot(s);
        fill(s, k, RESIDENT);
        ++st_.admitted;
        return s;
      }
    } else {
      const int r = coldest_resident();
      if (r >= 0 && touch_[k] > touch_[slots_[r].key]) {
        clear_slot(r);
        ++st_.evictions;
        fill(r, k, RESIDENT);
        ++st_.admitted;
        return r;
      }
    }
    int s = free_slot();
    if (s < 0) s = lru_transient();
    if (s < 0) return -1;
    if (slots_[s].state != FREE) ++st_.evictions;
    clear_slot(s);
    fill(s, k, TRANSIENT);
    ++st_.transient_loads;
    return s;
  }

  // Requested expert held as TRANSIENT in slot s: admit it without a copy.
  void promote(int s) {
    Slot& sl = slots_[s];
    if (res_ < cap_) {
      sl.state = RESIDENT;
      ++res_;
      ++st_.promotions;
      return;
    }
    const int r = coldest_resident();
    if (r >= 0 && touch_[sl.key] > touch_[slots_[r].key]) {
      slots_[r].state = TRANSIENT;  // keeps its expert, now evictable as a transient
      sl.state = RESIDENT;
      ++st_.promotions;
    }
  }

  int L_, E_, cap_;
  std::vector<Slot> slots_;
  std::vector<int32_t> where_;
  std::vector<uint32_t> touch_;
  int res_ = 0;
  int64_t epoch_ = 0;
  Stats st_;
};

}  // namespace moe
