"""The host-side expert cache (rl_cache_*) against a plain Python model of
the same policy: least recently used replacement, every hit of a selection
reserved before any victim is chosen, free slots used before any eviction,
the selection's slots most recently used on commit (first id most recent),
abort restoring every key to its slot.  Random selections drive both and
must agree on every slot, load flag, evicted key, generation and count.
No GPU is involved."""
import numpy as np
import pytest

from quantized_routed_expert_rl_amd import binding as B


class ModelLRU:
    """Recency as a Python list of slots, most recent first."""

    def __init__(self, n_slots, L, E):
        self.E = E
        self.order = list(range(n_slots))        # slot 0 is used first when all are free
        self.order.reverse()                     # ... so it sits at the least recent end
        self.key_of = [-1] * n_slots
        self.slot_of = {}
        self.gen = [0] * n_slots
        self.stats = dict(reservations=0, hits=0, misses=0, evictions=0, aborts=0)
        self.open = None

    def insert(self, layer, expert, slot):
        key = layer * self.E + expert
        self.slot_of[key] = slot
        self.key_of[slot] = key
        self.order.remove(slot)
        self.order.insert(0, slot)

    def reserve(self, layer, ids, exclude=-1):
        self.stats["reservations"] += 1
        keys = [layer * self.E + int(e) for e in ids]
        saved = (list(self.order), list(self.key_of), dict(self.slot_of))
        held = []
        slots = [self.slot_of.get(k, -1) for k in keys]
        for s in slots:
            if s >= 0 and s not in held:
                held.append(s)
        free = [s for s in self.order if s not in held
                and (self.key_of[s] < 0 or self.key_of[s] // self.E != exclude)]
        if len({k for k, s in zip(keys, slots) if s < 0}) > len(free):
            self.stats["aborts"] += 1            # refused before anything changes
            return None
        load, evicted = [0] * len(keys), [-1] * len(keys)
        for i, k in enumerate(keys):
            if slots[i] >= 0:
                self.stats["hits"] += 1
                continue
            if k in self.slot_of:
                slots[i] = self.slot_of[k]
                continue
            if not free:
                self.order, self.key_of, self.slot_of = saved
                self.stats["aborts"] += 1
                return None
            v = free.pop()                       # least recent unheld slot
            old = self.key_of[v]
            if old >= 0:
                del self.slot_of[old]
                self.stats["evictions"] += 1
            self.key_of[v] = k
            self.slot_of[k] = v
            self.gen[v] += 1
            self.stats["misses"] += 1
            held.append(v)
            slots[i], load[i], evicted[i] = v, 1, old
        self.open = (held, saved)
        return sum(load), slots, load, evicted, [self.gen[s] for s in slots]

    def touch(self, layer, ids):
        res = [self.slot_of[layer * self.E + int(e)] for e in ids
               if layer * self.E + int(e) in self.slot_of]
        self.order = res + [s for s in self.order if s not in res]
        return len(res)

    def commit(self):
        held, _ = self.open
        self.order = held + [s for s in self.order if s not in held]
        self.open = None

    def abort(self):
        held, (order, key_of, slot_of) = self.open
        self.key_of, self.slot_of = key_of, slot_of
        rest = [s for s in order if s not in held]
        self.order = ([s for s in held if self.key_of[s] >= 0] + rest
                      + [s for s in held if self.key_of[s] < 0])
        self.stats["aborts"] += 1
        self.open = None

    def table(self, L):
        t = np.full((L, self.E), -1, np.int32)
        for k, s in self.slot_of.items():
            t[k // self.E, k % self.E] = s
        return t


@pytest.mark.parametrize("n_slots,L,E,k,seed", [(8, 2, 16, 3, 0), (40, 4, 64, 8, 1),
                                                (12, 3, 20, 4, 2), (100, 6, 128, 10, 3)])
def test_cache_matches_model(n_slots, L, E, k, seed):
    rng = np.random.default_rng(seed)
    c, m = B.ExpertCache(n_slots, L, E), ModelLRU(n_slots, L, E)
    # seed part of the pool from a residency table
    for s, key in enumerate(rng.choice(L * E, n_slots // 2, replace=False)):
        c.insert(int(key) // E, int(key) % E, s)
        m.insert(int(key) // E, int(key) % E, s)
    pop = rng.permutation(E)                     # skewed selections: some experts hot
    for step in range(300):
        layer = int(rng.integers(L))
        p = 1.0 / (np.arange(E) + 1.0) ** 1.1
        ids = pop[rng.choice(E, k, replace=False, p=p / p.sum())].astype(np.int32)
        # a third of the reservations exclude another layer's slots as victims
        excl = int(rng.integers(L)) if rng.random() < 0.33 else -1
        got = c.reserve(layer, ids, exclude_layer=excl, raw=True)
        want = m.reserve(layer, ids, excl)
        if want is None:                         # too few slots qualify: refused, unchanged
            assert got[0] == B.RL_E_RANGE, step
            assert np.array_equal(c.table(), m.table(L)), step
            continue
        assert got[0] == want[0]
        for a, b in zip(got[1:], want[1:]):
            assert list(a) == list(b), step
        if rng.random() < 0.1:
            c.abort()
            m.abort()
        else:
            c.commit()
            m.commit()
        if rng.random() < 0.3:                   # a layer the device served from residents
            other = pop[rng.choice(E, k, replace=False)].astype(np.int32)
            lt = int(rng.integers(L))
            assert c.touch(lt, other) == m.touch(lt, other)
        assert np.array_equal(c.table(), m.table(L)), step
    assert c.stats() == m.stats
    assert m.stats["evictions"] > 0 and m.stats["hits"] > 0


def test_hits_are_never_evicted_by_their_own_selection():
    # 3 slots, all resident; a selection of one hit and two misses must
    # evict the two other slots, not the hit, even though it is the least
    # recently used
    c = B.ExpertCache(3, 1, 8)
    for s, e in enumerate([5, 6, 7]):
        c.insert(0, e, s)                        # 7 most recent, 5 least
    n, slots, load, evicted, gens = c.reserve(0, [5, 1, 2])
    assert n == 2 and slots[0] == 0 and list(load) == [0, 1, 1]
    assert sorted(evicted[1:].tolist()) == [6, 7]
    c.commit()
    assert c.lookup(0, 6) == -1 and c.lookup(0, 7) == -1 and c.lookup(0, 5) == 0


def test_selection_larger_than_the_pool_is_refused_and_rolled_back():
    c = B.ExpertCache(2, 1, 8)
    c.insert(0, 3, 0)
    before = c.table().copy()
    with pytest.raises(B.RlError):
        c.reserve(0, [1, 2, 3])                  # two misses, one free slot outside the selection
    assert np.array_equal(c.table(), before)
    assert c.stats()["aborts"] == 1
    n, *_ = c.reserve(0, [1, 3])                 # the cache is usable afterwards
    assert n == 1
    c.commit()


def test_excluded_layer_keeps_its_slots():
    # 4 slots: layer 0 holds experts 1, 2 (least recent), layer 1 holds 3, 4;
    # a layer-2 reservation that excludes layer 0 must evict layer 1's slots
    c = B.ExpertCache(4, 3, 8)
    for s, (l, e) in enumerate([(0, 1), (0, 2), (1, 3), (1, 4)]):
        c.insert(l, e, s)
    n, slots, load, evicted, gens = c.reserve(2, [5, 6], exclude_layer=0)
    assert n == 2 and sorted(slots.tolist()) == [2, 3]
    assert sorted(evicted.tolist()) == [1 * 8 + 3, 1 * 8 + 4]
    c.commit()
    assert c.lookup(0, 1) == 0 and c.lookup(0, 2) == 1
    # three misses, only the two layer-2 slots... all remaining victims are
    # layer 0's or the selection's own: refused, nothing changes
    before = c.table().copy()
    n, *_ = c.reserve(1, [0, 1, 2], exclude_layer=0, raw=True)
    assert n == B.RL_E_RANGE and np.array_equal(c.table(), before)
    # without the exclusion the same reservation evicts layer 0's experts
    n, slots, load, evicted, gens = c.reserve(1, [0, 1], exclude_layer=-1)
    assert n == 2 and sorted(evicted.tolist()) == [1, 2]
    c.commit()


def test_generations_count_loads_per_slot():
    c = B.ExpertCache(1, 2, 4)
    assert c.generation(0) == 0
    for i, e in enumerate([0, 1, 1, 2]):
        n, slots, load, evicted, gens = c.reserve(i % 2, [e])
        c.commit()
    # loads: (0,0) gen 1, (1,1) gen 2, (0,1) gen 3, (1,2) gen 4
    assert c.generation(0) == 4 and gens[0] == 4


def test_errors():
    c = B.ExpertCache(4, 2, 8)
    with pytest.raises(B.RlError):
        c.reserve(2, [0])                        # layer out of range
    with pytest.raises(B.RlError):
        c.reserve(0, [8])                        # expert out of range
    c.reserve(0, [1])
    with pytest.raises(B.RlError):
        c.reserve(0, [2])                        # a reservation is already open
    with pytest.raises(B.RlError):
        c.insert(1, 1, 3)                        # no inserts while it is open
    c.commit()
    with pytest.raises(B.RlError):
        c.insert(0, 1, 3)                        # already resident
    assert B.lib.rl_cache_create(0, 1, 1) is None
    assert B.lib.rl_cache_lookup(None, 0, 0) == -1
