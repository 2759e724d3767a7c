// Host-side expert cache over the device slot pool (host code only).
//
// The residency table maps (layer, expert) to a pool slot; when a layer's
// selection names an expert that is not resident, the host loads it into a
// slot and updates the table ("Red Lite dev21 - GPU-routed decode", "What
// changed": the residency table is maintained on every LRU commit and abort,
// and a reservation reports the key a miss evicts; "Red Lite dev23", "What
// changed": per-slot load generations checked at release).  The replacement
// policy is least-recently-used, with every hit of a selection reserved
// before any victim is chosen, so a selection never evicts one of its own
// experts ("Red Lite dev20 - batched prompt ingestion", LRU fix: hits are
// reserved first; resident keys are found through an index instead of a
// scan).  Here the index is a dense [layers x experts] array, which the
// key space allows.
//
// Recency is an intrusive doubly linked list over slots, most recent at the
// head; free slots start at the tail so they are used before any resident
// expert is evicted.  Slots reserved by the open reservation are taken out
// of the list (pinned) until commit or abort.  Not thread-safe.
#include <cstdint>
#include <new>
#include <vector>

#include "rl_moe.h"

struct rl_cache {
  int32_t n_slots, n_layers, n_experts;
  std::vector<int32_t> key_of_slot;   // (layer * E + expert) held by a slot, -1 free
  std::vector<int32_t> slot_of_key;   // [L * E] slot of a key, -1 not resident
  std::vector<int32_t> prev, next;    // recency list, -1 ends it
  std::vector<uint8_t> pinned;
  std::vector<uint32_t> gen;          // loads into each slot so far
  std::vector<int32_t> per_layer;     // resident experts of each layer
  int32_t head = -1, tail = -1;
  // the open reservation: pinned slots in order, and (slot, previous key, new key) of each load
  std::vector<int32_t> held;
  struct Load { int32_t slot, old_key, new_key; };
  std::vector<Load> loads;
  int64_t stats[5] = {0, 0, 0, 0, 0};  // reservations, hits, misses, evictions, aborts
};

namespace {

void unlink(rl_cache* c, int32_t s) {
  const int32_t p = c->prev[s], n = c->next[s];
  if (p >= 0) c->next[p] = n; else c->head = n;
  if (n >= 0) c->prev[n] = p; else c->tail = p;
  c->prev[s] = c->next[s] = -1;
}

void push_head(rl_cache* c, int32_t s) {
  c->prev[s] = -1;
  c->next[s] = c->head;
  if (c->head >= 0) c->prev[c->head] = s; else c->tail = s;
  c->head = s;
}

void push_tail(rl_cache* c, int32_t s) {
  c->next[s] = -1;
  c->prev[s] = c->tail;
  if (c->tail >= 0) c->next[c->tail] = s; else c->head = s;
  c->tail = s;
}

bool valid_key(const rl_cache* c, int32_t layer, int32_t expert) {
  return layer >= 0 && layer < c->n_layers && expert >= 0 && expert < c->n_experts;
}

// Undo the open reservation: keys return to their slots; reserved slots
// that hold a key again go to the head (the first reserved most recent),
// slots that are free again to the tail.
void rollback(rl_cache* c) {
  for (auto it = c->loads.rbegin(); it != c->loads.rend(); ++it) {
    c->slot_of_key[it->new_key] = -1;
    c->key_of_slot[it->slot] = it->old_key;
    c->per_layer[it->new_key / c->n_experts] -= 1;
    if (it->old_key >= 0) {
      c->slot_of_key[it->old_key] = it->slot;
      c->per_layer[it->old_key / c->n_experts] += 1;
    }
  }
  for (auto it = c->held.rbegin(); it != c->held.rend(); ++it) {
    c->pinned[*it] = 0;
    if (c->key_of_slot[*it] >= 0) push_head(c, *it);
  }
  for (int32_t s : c->held)
    if (c->key_of_slot[s] < 0) push_tail(c, s);
  c->held.clear();
  c->loads.clear();
}

}  // namespace

extern "C" {

rl_cache* rl_cache_create(int32_t n_slots, int32_t n_layers, int32_t n_experts) {
  if (n_slots < 1 || n_layers < 1 || n_experts < 1 ||
      int64_t(n_layers) * n_experts > (int64_t(1) << 30))
    return nullptr;
  rl_cache* c = new (std::nothrow) rl_cache;
  if (!c) return nullptr;
  c->n_slots = n_slots;
  c->n_layers = n_layers;
  c->n_experts = n_experts;
  c->key_of_slot.assign(n_slots, -1);
  c->slot_of_key.assign(size_t(n_layers) * n_experts, -1);
  c->prev.assign(n_slots, -1);
  c->next.assign(n_slots, -1);
  c->pinned.assign(n_slots, 0);
  c->gen.assign(n_slots, 0);
  c->per_layer.assign(n_layers, 0);
  for (int32_t s = 0; s < n_slots; ++s) push_head(c, s);   // slot 0 least recent: used first
  return c;
}

void rl_cache_destroy(rl_cache* c) { delete c; }

int rl_cache_insert(rl_cache* c, int32_t layer, int32_t expert, int32_t slot) {
  if (!c) return RL_E_INVAL;
  if (!valid_key(c, layer, expert) || slot < 0 || slot >= c->n_slots) return RL_E_RANGE;
  if (!c->held.empty()) return RL_E_INVAL;            // a reservation is open
  const int32_t key = layer * c->n_experts + expert;
  if (c->slot_of_key[key] >= 0 || c->key_of_slot[slot] >= 0) return RL_E_INVAL;
  c->slot_of_key[key] = slot;
  c->key_of_slot[slot] = key;
  c->per_layer[layer] += 1;
  unlink(c, slot);
  push_head(c, slot);
  return RL_OK;
}

int32_t rl_cache_lookup(const rl_cache* c, int32_t layer, int32_t expert) {
  if (!c || !valid_key(c, layer, expert)) return -1;
  return c->slot_of_key[size_t(layer) * c->n_experts + expert];
}

int rl_cache_reserve(rl_cache* c, int32_t layer, const int32_t* ids, int32_t k, int32_t* slots,
                     int32_t* load, int32_t* evicted, uint32_t* gens) {
  return rl_cache_reserve_excluding(c, layer, ids, k, -1, slots, load, evicted, gens);
}

int rl_cache_reserve_excluding(rl_cache* c, int32_t layer, const int32_t* ids, int32_t k,
                               int32_t exclude_layer, int32_t* slots, int32_t* load,
                               int32_t* evicted, uint32_t* gens) {
  if (!c || !ids || !slots || !load || !evicted) return RL_E_INVAL;
  if (!c->held.empty()) return RL_E_INVAL;            // commit or abort the previous one first
  if (layer < 0 || layer >= c->n_layers || k < 1) return RL_E_RANGE;
  for (int32_t i = 0; i < k; ++i)
    if (ids[i] < 0 || ids[i] >= c->n_experts) return RL_E_RANGE;
  c->stats[0] += 1;
  // refuse, changing nothing, a selection with more distinct misses than
  // slots that may be victims: outside its distinct hits and not holding an
  // expert of exclude_layer (the hits are the layer's own experts)
  int32_t n_hit = 0, n_miss = 0;
  for (int32_t i = 0; i < k; ++i) {
    bool repeat = false;
    for (int32_t j = 0; j < i && !repeat; ++j) repeat = ids[j] == ids[i];
    if (repeat) continue;
    if (c->slot_of_key[size_t(layer) * c->n_experts + ids[i]] >= 0) ++n_hit; else ++n_miss;
  }
  int32_t n_victims = c->n_slots - n_hit;
  if (exclude_layer == layer)
    n_victims = c->n_slots - c->per_layer[layer];
  else if (exclude_layer >= 0 && exclude_layer < c->n_layers)
    n_victims -= c->per_layer[exclude_layer];
  if (n_miss > n_victims) {
    c->stats[4] += 1;
    return RL_E_RANGE;
  }
  // hits first: every resident expert of the selection is pinned before
  // any victim is chosen
  for (int32_t i = 0; i < k; ++i) {
    const int32_t key = layer * c->n_experts + ids[i];
    const int32_t s = c->slot_of_key[key];
    load[i] = 0;
    evicted[i] = -1;
    slots[i] = s;
    if (s >= 0 && !c->pinned[s]) {
      c->pinned[s] = 1;
      unlink(c, s);
      c->held.push_back(s);
    }
  }
  int32_t n_loads = 0;
  for (int32_t i = 0; i < k; ++i) {
    if (slots[i] >= 0) {
      c->stats[1] += 1;
      continue;
    }
    const int32_t key = layer * c->n_experts + ids[i];
    const int32_t again = c->slot_of_key[key];        // a repeated id, loaded above
    if (again >= 0) {
      slots[i] = again;
      continue;
    }
    // least recently used, unpinned, and not holding an expert of exclude_layer
    int32_t v = c->tail;
    while (v >= 0 && c->key_of_slot[v] >= 0 && c->key_of_slot[v] / c->n_experts == exclude_layer)
      v = c->prev[v];
    if (v < 0) {                                      // not reached: counted above
      rollback(c);
      c->stats[4] += 1;
      return RL_E_RANGE;
    }
    unlink(c, v);
    c->pinned[v] = 1;
    c->held.push_back(v);
    const int32_t old = c->key_of_slot[v];
    if (old >= 0) {
      c->slot_of_key[old] = -1;
      c->per_layer[old / c->n_experts] -= 1;
      c->stats[3] += 1;
    }
    c->per_layer[layer] += 1;
    c->loads.push_back({v, old, key});
    c->key_of_slot[v] = key;
    c->slot_of_key[key] = v;
    c->gen[v] += 1;
    c->stats[2] += 1;
    slots[i] = v;
    load[i] = 1;
    evicted[i] = old;
    ++n_loads;
  }
  if (gens)
    for (int32_t i = 0; i < k; ++i) gens[i] = c->gen[slots[i]];
  return n_loads;
}

int rl_cache_touch(rl_cache* c, int32_t layer, const int32_t* ids, int32_t k) {
  if (!c || !ids) return RL_E_INVAL;
  if (!c->held.empty()) return RL_E_INVAL;
  if (layer < 0 || layer >= c->n_layers || k < 0) return RL_E_RANGE;
  int32_t n = 0;
  for (int32_t i = k - 1; i >= 0; --i) {              // the first id ends most recent
    if (ids[i] < 0 || ids[i] >= c->n_experts) return RL_E_RANGE;
    const int32_t s = c->slot_of_key[size_t(layer) * c->n_experts + ids[i]];
    if (s < 0) continue;
    unlink(c, s);
    push_head(c, s);
    ++n;
  }
  return n;
}

int rl_cache_commit(rl_cache* c) {
  if (!c) return RL_E_INVAL;
  // most recently used: the selection's slots, the first id at the head
  for (auto it = c->held.rbegin(); it != c->held.rend(); ++it) {
    c->pinned[*it] = 0;
    push_head(c, *it);
  }
  c->held.clear();
  c->loads.clear();
  return RL_OK;
}

int rl_cache_abort(rl_cache* c) {
  if (!c) return RL_E_INVAL;
  if (!c->held.empty()) c->stats[4] += 1;
  rollback(c);
  return RL_OK;
}

uint32_t rl_cache_generation(const rl_cache* c, int32_t slot) {
  if (!c || slot < 0 || slot >= c->n_slots) return 0;
  return c->gen[slot];
}

int rl_cache_table(const rl_cache* c, int32_t* table) {
  if (!c || !table) return RL_E_INVAL;
  for (size_t i = 0; i < c->slot_of_key.size(); ++i) table[i] = c->slot_of_key[i];
  return RL_OK;
}

int rl_cache_stats(const rl_cache* c, int64_t* out) {
  if (!c || !out) return RL_E_INVAL;
  for (int i = 0; i < 5; ++i) out[i] = c->stats[i];
  return RL_OK;
}

}  // extern "C"
