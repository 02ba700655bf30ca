"""Precision tiers in the expert pool, on the host (bookkeeping-only pools).

Reading (the pages list int8, int4 and int2 kernels with per-row scales and
name no tiering policy): an expert may carry a second, narrower block; with
demotion on, a refill of an unpinned expert whose full-width block finds no
free extent large enough loads the narrower block, evicting for that size
only; the expert keeps its width until evicted; pinned experts load at full
width, and pinning re-loads a demoted copy.

The residency and width of every expert after every call are checked against
an independent reference simulation that carries its own first-fit allocator
with coalescing (widths differ, so placement decides what fits), and the
statistics against the simulation's counts.
"""
from collections import OrderedDict

import numpy as np
import pytest

torch = pytest.importorskip("torch")

H, I = 256, 128


@pytest.fixture(scope="module")
def moe():
    import quantized_moe_expert_sigmoid_amd as m
    m.lib()
    return m


def nbytes(moe, bits):
    return moe.moe_expert_block_layout(bits, H, I)[0]


class RefTierPool:
    """Reference model: first-fit slab, one LRU over unpinned residents,
    demotion of refills under pressure."""

    def __init__(self, capacity, sizes, demote):
        self.cap = capacity // 256 * 256
        self.sizes = sizes
        self.demote = demote
        self.reg = {}          # key -> (bits, alt_bits or 0, pin)
        self.res = {}          # key -> (off, length, bits)
        self.lru = OrderedDict()
        self.last = {}
        self.free = [[0, self.cap]]
        self.epoch = 0
        self.hits = self.misses = self.h2d = 0
        self.dloads = self.duses = self.saved = 0

    def _alloc(self, n):
        for f in self.free:  # kept sorted by offset
            if f[1] >= n:
                off = f[0]
                f[0] += n
                f[1] -= n
                if f[1] == 0:
                    self.free.remove(f)
                return off
        return None

    def _release(self, off, n):
        self.free.append([off, n])
        self.free.sort()
        merged = []
        for f in self.free:
            if merged and merged[-1][0] + merged[-1][1] == f[0]:
                merged[-1][1] += f[1]
            else:
                merged.append(f)
        self.free = merged

    def _evict(self, key):
        off, n, _ = self.res.pop(key)
        self.lru.pop(key, None)
        self._release(off, n)

    def _refill(self, key, ep, protect):
        bits, alt, pin = self.reg[key]
        full = self.sizes[bits]
        narrow = self.demote and alt and not pin and not any(f[1] >= full for f in self.free)
        b = alt if narrow else bits
        n = self.sizes[b]
        while True:
            off = self._alloc(n)
            if off is not None:
                break
            if not self.lru or self.last[next(iter(self.lru))] >= protect:
                raise RuntimeError("pool full")
            self._evict(next(iter(self.lru)))
        self.res[key] = (off, n, b)
        self.last[key] = ep
        if not pin:
            self.lru[key] = True
        self.h2d += n
        if narrow:
            self.dloads += 1
            self.saved += full - n

    def call(self, layer, ids):
        self.epoch += 1
        ep = self.epoch
        keys = [(layer, e) for e in sorted(set(int(e) for e in np.asarray(ids).ravel()) - {-1})]
        for kk in keys:
            if kk not in self.res:
                continue
            bits, _, pin = self.reg[kk]
            if pin and self.res[kk][2] != bits:
                self._evict(kk)
                continue
            self.last[kk] = ep
            if not pin:
                self.lru.move_to_end(kk)
            self.hits += 1
            if self.res[kk][2] != bits:
                self.duses += 1
        for kk in keys:
            if kk in self.res:
                continue
            self._refill(kk, ep, ep)
            self.misses += 1
            if self.res[kk][2] != self.reg[kk][0]:
                self.duses += 1

    def width(self, key):
        return self.res[key][2] if key in self.res else 0


def build(moe, capacity, layers, E, demote, seed):
    """A pool and its reference with a mix of experts: int8 with an int4
    block, int4 with an int2 block, int4 alone, int2 alone, a few pinned."""
    rng = np.random.default_rng(seed)
    sizes = {b: nbytes(moe, b) for b in (8, 4, 2)}
    pool = moe.MoePool(None, capacity, layers, E, H, I)
    ref = RefTierPool(capacity, sizes, demote)
    for L in range(layers):
        for e in range(E):
            kind = rng.integers(0, 4)
            bits, alt = [(8, 4), (4, 2), (4, 0), (2, 0)][kind]
            pin = bool(rng.random() < 0.08) and bits != 8
            pool.register(L, e, bits, None, pin=pin)
            if alt:
                pool.register_alt(L, e, alt, None)
            ref.reg[(L, e)] = (bits, alt, pin)
    pool.set_demotion(demote)
    return pool, ref


@pytest.mark.parametrize("demote", [False, True])
@pytest.mark.parametrize("cap_blocks,E,k,layers,seed", [(7.3, 12, 3, 2, 0), (10.3, 12, 3, 2, 3), (11.0, 24, 4, 3, 1), (5.6, 10, 2, 1, 2)])
def test_tiers_match_reference(moe, demote, cap_blocks, E, k, layers, seed):
    capacity = int(cap_blocks * nbytes(moe, 4))
    pool, ref = build(moe, capacity, layers, E, demote, seed)
    rng = np.random.default_rng(100 + seed)
    zipf = 1.0 / np.arange(1, E + 1) ** 1.1
    zipf /= zipf.sum()
    n_demoted_seen = 0
    for step in range(400):
        L = int(rng.integers(0, layers))
        ids = rng.choice(E, size=k, replace=False, p=zipf).astype(np.int32)
        try:
            ref.call(L, ids)
        except RuntimeError:
            with pytest.raises(Exception):
                pool.prepare(L, ids[None, :])
            break
        pool.prepare(L, ids[None, :])
        assert pool.call_widths() == sum({1 << ref.width((L, int(e))) for e in ids}), step
        for LL in range(layers):
            for e in range(E):
                w = pool.resident_bits(LL, e)
                assert w == ref.width((LL, e)), (step, LL, e)
                n_demoted_seen += int(w != 0 and w != ref.reg[(LL, e)][0])
        st = pool.stats()
        assert (st["hits"], st["misses"], st["bytes_h2d"]) == (ref.hits, ref.misses, ref.h2d)
        ts = pool.tier_stats()
        assert (ts["demoted_loads"], ts["demoted_uses"], ts["bytes_saved"]) == (ref.dloads, ref.duses, ref.saved)
    if demote:
        assert n_demoted_seen > 0  # the case reached pressure
    else:
        assert pool.tier_stats()["demoted_loads"] == 0
    pool.close()


def uniform_pool(moe, slots4, E=8, alt=2, demote=True):
    pool = moe.MoePool(None, int(slots4 * nbytes(moe, 4)), 1, E, H, I)
    for e in range(E):
        pool.register(0, e, 4, None)
        pool.register_alt(0, e, alt, None)
    pool.set_demotion(demote)
    return pool


def test_full_width_while_room_then_narrow(moe):
    b4, b2 = nbytes(moe, 4), nbytes(moe, 2)
    pool = uniform_pool(moe, 3)
    pool.prepare(0, np.array([[0, 1, 2]], np.int32))  # room for all three at full width
    assert [pool.resident_bits(0, e) for e in range(3)] == [4, 4, 4]
    pool.prepare(0, np.array([[3]], np.int32))  # full: evicts 0, loads the int2 block in its place
    assert pool.resident_bits(0, 0) == 0 and pool.resident_bits(0, 3) == 2
    assert pool.tier_stats() == {"demoted_loads": 1, "demoted_uses": 1, "bytes_saved": b4 - b2}
    assert pool.stats()["bytes_h2d"] == 3 * b4 + b2
    pool.prepare(0, np.array([[4]], np.int32))  # the hole left beside 3 (b4 - b2) is too small: evicts 1
    assert pool.resident_bits(0, 1) == 0 and pool.resident_bits(0, 4) == 2
    pool.prepare(0, np.array([[3, 4]], np.int32))  # hits served by int2 copies
    assert pool.tier_stats()["demoted_uses"] == 4
    pool.close()


def test_demotion_off_and_pinned_stay_full_width(moe):
    pool = uniform_pool(moe, 2, demote=False)
    for e in range(5):
        pool.prepare(0, np.array([[e]], np.int32))
        assert pool.resident_bits(0, e) == 4
    assert pool.tier_stats()["demoted_loads"] == 0
    pool.close()
    pool = moe.MoePool(None, int(2.5 * nbytes(moe, 4)), 1, 4, H, I)
    pool.register(0, 0, 4, None, pin=True)
    pool.register_alt(0, 0, 2, None)
    for e in range(1, 4):
        pool.register(0, e, 4, None)
        pool.register_alt(0, e, 2, None)
    pool.set_demotion(True)
    pool.prepare(0, np.array([[1, 2]], np.int32))  # fills the room at full width
    pool.prepare(0, np.array([[0]], np.int32))  # pinned: full width, evicting one
    assert pool.resident_bits(0, 0) == 4
    pool.close()


def test_pin_hot_reloads_demoted_at_full_width(moe):
    pool = uniform_pool(moe, 3)
    pool.prepare(0, np.array([[0, 1, 2]], np.int32))
    pool.prepare(0, np.array([[3]], np.int32))  # 3 at int2
    pool.prepare(0, np.array([[4]], np.int32))  # 4 at int2 (latest call)
    assert pool.resident_bits(0, 3) == 2 and pool.resident_bits(0, 4) == 2
    counts = np.zeros((1, 8), np.uint64)
    counts[0, 3], counts[0, 4] = 5, 4
    assert pool.pin_hot(2 * nbytes(moe, 4), counts) == 2
    assert pool.resident_bits(0, 3) == 4  # re-loaded now
    assert pool.resident_bits(0, 4) == 2  # the latest call uses it: re-loaded at its next request
    m0 = pool.stats()["misses"]
    assert pool.prepare(0, np.array([[4]], np.int32)) == 1
    assert pool.resident_bits(0, 4) == 4 and pool.stats()["misses"] == m0 + 1
    for e in (5, 6, 7, 0):  # pinned experts survive the churn at full width
        pool.prepare(0, np.array([[e]], np.int32))
        assert pool.resident_bits(0, 3) == 4 and pool.resident_bits(0, 4) == 4
    pool.close()


def test_tier_errors(moe):
    pool = moe.MoePool(None, 4 * nbytes(moe, 8), 1, 4, H, I)
    with pytest.raises(Exception):
        pool.register_alt(0, 0, 2, None)  # no full-width block yet
    pool.register(0, 0, 4, None)
    pool.register(0, 1, 2, None)
    pool.register(0, 2, 8, None)
    with pytest.raises(Exception):
        pool.register_alt(0, 0, 4, None)  # not narrower
    with pytest.raises(Exception):
        pool.register_alt(0, 1, 2, None)  # int2 has nothing narrower
    with pytest.raises(Exception):
        pool.register_alt(0, 0, 2, None, nbytes=nbytes(moe, 2) + 256)  # wrong size
    with pytest.raises(Exception):
        pool.register_alt(0, 2, 8, None)
    pool.register_alt(0, 0, 2, None)
    pool.register_alt(0, 2, 4, None)
    with pytest.raises(Exception):
        pool.register_alt(0, 0, 2, None)  # twice
    with pytest.raises(Exception):
        pool.resident_bits(0, 9)
    assert pool.resident_bits(0, 0) == 0
    pool.close()
