"""Slot-table policy on the host (no GPU): the library's host-only table reports
each copy it would enqueue; a small independent LRU model predicts them."""
import numpy as np
import pytest

import expert_routed_ffn_amd as m
from expert_routed_ffn_amd import _lib


class LRUModel:
    """Least recently used over (layer, expert); misses in ascending expert id;
    free slots first, in ascending order."""

    def __init__(self, L, E, n):
        self.E, self.n = E, n
        self.order = list(range(n))  # LRU first
        self.owner = [None] * n
        self.where = {}

    def _touch(self, s):
        self.order.remove(s)
        self.order.append(s)

    def resolve(self, layer, active):
        copies = []
        for e in active:
            s = self.where.get((layer, e))
            if s is not None:
                self._touch(s)
        for e in sorted(set(active)):
            if (layer, e) in self.where:
                continue
            s = self.order[0]
            if self.owner[s] is not None:
                del self.where[self.owner[s]]
            self.owner[s] = (layer, e)
            self.where[(layer, e)] = s
            self._touch(s)
            copies.append((s, layer, e))
        return copies


def test_worked_sequence():
    t = m.HostSlotTable(2, 8, 4)
    t.resolve(0, [1, 3])
    assert t.copies == [(0, 0, 1), (1, 0, 3)]
    t.resolve(0, [3, 5])
    assert t.copies[2:] == [(2, 0, 5)]
    t.resolve(1, [2, 0])
    assert t.copies[3:] == [(3, 1, 0), (0, 1, 2)]  # slot 0 (layer 0, expert 1) was least recently used
    mp = t.map_host().reshape(2, 8)
    assert mp[0, 1] == -1 and mp[0, 3] == 1 and mp[0, 5] == 2 and mp[1, 0] == 3 and mp[1, 2] == 0
    st = t.stats()
    assert st["hits"] == 1 and st["misses"] == 5 and st["evictions"] == 1 and st["resolves"] == 3


def test_capacity_error():
    t = m.HostSlotTable(1, 16, 4)
    with pytest.raises(m.MoeError) as ei:
        t.resolve(0, [0, 1, 2, 3, 4])
    assert ei.value.status == _lib.MOE_ECAPACITY
    with pytest.raises(m.MoeError):
        t.resolve(0, [16])


@pytest.mark.parametrize("L,E,n,seed", [(4, 64, 32, 0), (48, 512, 256, 1), (3, 16, 10, 2)])
def test_matches_lru_model_and_invariants(L, E, n, seed):
    rng = np.random.default_rng(seed)
    t = m.HostSlotTable(L, E, n)
    model = LRUModel(L, E, n)
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    p /= p.sum()
    for step in range(60):
        for layer in range(L):
            act = sorted(set(rng.choice(E, size=min(n, 10), p=p).tolist()))
            before = len(t.copies)
            t.resolve(layer, act)
            assert t.copies[before:] == model.resolve(layer, act)
            mp = t.map_host().reshape(L, E)
            for e in act:  # every active expert is resident after the resolve
                assert mp[layer, e] >= 0
            used = mp[mp >= 0]
            assert len(used) == len(set(used.tolist())) <= n  # a slot holds at most one expert
    st = t.stats()
    assert st["misses"] == len(t.copies) and st["bytes_h2d"] == 256 * len(t.copies)


def test_all_miss_when_capacity_equals_active_set():
    t = m.HostSlotTable(2, 32, 4)
    for step in range(5):
        t.resolve(step % 2, [4 * step % 32, (4 * step + 1) % 32, (4 * step + 2) % 32, (4 * step + 3) % 32])
    st = t.stats()
    assert st["hits"] == 0 and st["misses"] == 20


def test_device_table_rejects_bad_arguments_without_gpu():
    import ctypes
    h = ctypes.c_void_p()
    fake = ctypes.c_void_p(0x1000)
    L = _lib.lib
    assert L.moe_slot_table_create(2, 8, 4, 1000, fake, fake, fake, None, ctypes.byref(h)) == _lib.MOE_EINVAL
    assert L.moe_slot_table_create(0, 8, 4, 1024, fake, fake, fake, None, ctypes.byref(h)) == _lib.MOE_EINVAL
    assert L.moe_slot_table_create(2, 8, 4, 1024, None, fake, fake, None, ctypes.byref(h)) == _lib.MOE_EINVAL
