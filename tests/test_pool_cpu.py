"""Expert pool policy on the host (bookkeeping-only pools: no device needed).

The pool's residency decisions are checked against an independent reference
simulation of the documented policy: one least-recently-used order over every
layer's resident experts; a call's hits refresh their position (ascending
expert id), then its misses are inserted (ascending id), each evicting from
the cold end experts the call does not need; pinned experts are never
evicted. With equal block sizes the slab holds floor(capacity / block) blocks
whatever the placement, so the reference needs no allocator; mixed widths are
checked through invariants.
"""
from collections import OrderedDict

import numpy as np
import pytest

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def moe():
    import quantized_moe_expert_sigmoid_amd as m
    m.lib()
    return m


H, I = 256, 128


def block(moe, bits):
    return moe.moe_expert_block_layout(bits, H, I)[0]


class RefLRU:
    """Reference model of the pool policy for equal-size blocks."""

    def __init__(self, slots, pinned=()):
        self.slots = slots
        self.pinned = set(pinned)
        self.pinned_res = set()
        self.lru = OrderedDict()
        self.hits = self.misses = 0

    def resident(self, key):
        return key in self.lru or key in self.pinned_res

    def call(self, layer, ids):
        want = sorted(set(int(e) for e in np.asarray(ids).ravel()))
        keys = [(layer, e) for e in want]
        for kk in keys:  # hits
            if kk in self.pinned_res:
                self.hits += 1
            elif kk in self.lru:
                self.lru.move_to_end(kk)
                self.hits += 1
        used = set(keys)
        miss = 0
        for kk in keys:
            if self.resident(kk):
                continue
            while len(self.lru) + len(self.pinned_res) >= self.slots:
                victim = next(iter(self.lru)) if self.lru else None
                if victim is None or victim in used:
                    raise RuntimeError("pool full")
                self.lru.pop(victim)
            if kk in self.pinned:
                self.pinned_res.add(kk)
            else:
                self.lru[kk] = True
            self.misses += 1
            miss += 1
        return miss


@pytest.mark.parametrize("slots,E,k,layers,seed", [(5, 16, 2, 3, 0), (12, 32, 4, 2, 1), (8, 8, 3, 4, 2)])
def test_lru_matches_reference(moe, slots, E, k, layers, seed):
    rng = np.random.default_rng(seed)
    b = block(moe, 4)
    pool = moe.MoePool(None, slots * b + 100, layers, E, H, I)
    for L in range(layers):
        for e in range(E):
            pool.register(L, e, 4, None)
    ref = RefLRU(slots)
    for step in range(400):
        L = int(rng.integers(layers))
        T = int(rng.integers(1, 3))
        # skewed popularity so that hits happen
        ids = np.stack([rng.choice(E, size=k, replace=False, p=None if step % 3 else
                                   np.arange(E, 0, -1) / np.arange(E, 0, -1).sum()) for _ in range(T)])
        if len(set(ids.ravel())) > slots:
            continue
        got = pool.prepare(L, ids.astype(np.int32))
        assert got == ref.call(L, ids), step
        for LL in range(layers):
            for e in range(E):
                assert pool.resident(LL, e) == ref.resident((LL, e)), (step, LL, e)
    st = pool.stats()
    assert (st["hits"], st["misses"]) == (ref.hits, ref.misses)
    assert st["bytes_h2d"] == ref.misses * b
    pool.close()


def test_pinned_experts_stay(moe):
    b = block(moe, 4)
    E = 16
    pool = moe.MoePool(None, 6 * b, 1, E, H, I)
    for e in range(E):
        pool.register(0, e, 4, None, pin=e in (3, 7))
    ref = RefLRU(6, pinned=[(0, 3), (0, 7)])
    rng = np.random.default_rng(5)
    for step in range(300):
        ids = rng.choice(E, size=(1, 3), replace=False).astype(np.int32)
        assert pool.prepare(0, ids) == ref.call(0, ids)
        if step > 50:
            for e in (3, 7):
                assert pool.resident(0, e) == ref.resident((0, e))
    assert pool.resident(0, 3) and pool.resident(0, 7)  # both were requested at some point and never left
    pool.close()


def test_mixed_widths_invariants(moe):
    b4, b2, b8 = block(moe, 4), block(moe, 2), block(moe, 8)
    cap = 3 * b8 + b4
    E, layers = 24, 2
    widths = {}
    pool = moe.MoePool(None, cap, layers, E, H, I)
    rng = np.random.default_rng(7)
    for L in range(layers):
        for e in range(E):
            widths[(L, e)] = int(rng.choice([8, 4, 2]))
            pool.register(L, e, widths[(L, e)], None)
    size = {8: b8, 4: b4, 2: b2}
    refused = 0
    for step in range(500):
        L = int(rng.integers(layers))
        ids = rng.choice(E, size=(2, 2), replace=False).astype(np.int32)
        want = set(ids.ravel().tolist())
        before = pool.stats()
        was = {e: pool.resident(L, e) for e in want}
        try:
            m = pool.prepare(L, ids)
        except moe.MoeError as ex:  # fragmentation or a too-large working set may refuse a call
            assert ex.status == moe.MOE_EPOOL
            refused += 1
            continue
        after = pool.stats()
        assert after["misses"] - before["misses"] == m
        assert after["hits"] - before["hits"] == len(want) - m
        assert m == sum(1 for e in want if not was[e])
        assert after["bytes_h2d"] - before["bytes_h2d"] == sum(size[widths[(L, e)]] for e in want if not was[e])
        for e in want:
            assert pool.resident(L, e)
        used = sum(size[widths[(LL, e)]] for LL in range(layers) for e in range(E) if pool.resident(LL, e))
        assert used <= cap
    assert refused < 250


def test_pool_errors(moe):
    b = block(moe, 4)
    pool = moe.MoePool(None, 2 * b, 2, 8, H, I)
    for e in range(8):
        pool.register(0, e, 4, None)
    with pytest.raises(moe.MoeError) as ex:
        pool.register(0, 1, 4, None)  # twice
    assert ex.value.status == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError):
        pool.register(2, 0, 4, None)  # layer out of range
    with pytest.raises(moe.MoeError):
        pool.register(1, 0, 3, None)  # bits
    with pytest.raises(moe.MoeError):
        pool.register(1, 0, 4, None, nbytes=b - 256)  # wrong block size
    with pytest.raises(moe.MoeError) as ex:
        pool.prepare(0, np.array([[0, 9]], np.int32))  # id out of range
    assert ex.value.status == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError) as ex:
        pool.prepare(1, np.array([[0, 1]], np.int32))  # not registered
    assert ex.value.status == moe.MOE_EINVAL
    with pytest.raises(moe.MoeError) as ex:
        pool.prepare(0, np.array([[0, 1], [2, 3]], np.int32))  # 4 experts, room for 2
    assert ex.value.status == moe.MOE_EPOOL
    # the books stay usable after a refusal
    assert pool.prepare(0, np.array([[4, 5]], np.int32)) in (1, 2)
    assert pool.resident(0, 4) and pool.resident(0, 5)
    assert pool.prepare(0, np.zeros((0, 2), np.int32)) == 0  # an empty call
    with pytest.raises(moe.MoeError):
        moe.MoePool(None, 2 * b, 1, 8, 100, I)  # H not a multiple of 64
    pool.close()


def test_capacity_planning_monotone(moe):
    """More capacity never lowers the hit count on the same trace (LRU is a
    stack algorithm for equal block sizes)."""
    b = block(moe, 4)
    rng = np.random.default_rng(11)
    E, layers, k = 64, 4, 8
    p = 1.0 / np.arange(1, E + 1) ** 1.1
    p /= p.sum()
    trace = [(t % layers, rng.choice(E, size=(1, k), replace=False, p=p).astype(np.int32)) for t in range(1200)]
    hits = []
    for slots in (16, 32, 64, 128, 256):
        pool = moe.MoePool(None, slots * b, layers, E, H, I)
        for L in range(layers):
            for e in range(E):
                pool.register(L, e, 4, None)
        for L, ids in trace:
            pool.prepare(L, ids)
        hits.append(pool.stats()["hits"])
        pool.close()
    assert all(a <= b_ for a, b_ in zip(hits, hits[1:])), hits
    assert hits[-1] >= 1200 * k - layers * E  # everything fits: only first touches miss


# --------------------------------------------------------------------------
# read-ahead, usage counts and usage-learned pinning
# --------------------------------------------------------------------------

def make_pool(moe, slots, layers=1, E=16):
    b = block(moe, 4)
    pool = moe.MoePool(None, slots * b, layers, E, H, I)
    for L in range(layers):
        for e in range(E):
            pool.register(L, e, 4, None)
    return pool


def test_prefetch_then_prepare_hits(moe):
    pool = make_pool(moe, 8)
    assert pool.prepare(0, np.array([[0, 1]], np.int32)) == 2
    assert pool.prefetch(0, [2, 3, -1, 1]) == 2  # 1 is already resident, -1 names no expert
    assert pool.resident(0, 2) and pool.resident(0, 3)
    assert pool.prepare(0, np.array([[2, 3]], np.int32)) == 0
    assert pool.prefetch_stats() == {"issued": 2, "used": 2}
    st = pool.stats()
    assert (st["hits"], st["misses"]) == (2, 2)
    pool.close()


def test_prefetch_never_evicts_the_latest_call(moe):
    pool = make_pool(moe, 4)
    pool.prepare(0, np.array([[0, 1, 2, 3]], np.int32))  # fills the slab
    assert pool.prefetch(0, [4, 5]) == 0  # every resident expert belongs to the latest call
    assert all(pool.resident(0, e) for e in range(4)) and not pool.resident(0, 4)
    pool.prepare(0, np.array([[2, 3]], np.int32))  # 0 and 1 now belong to an older call
    assert pool.prefetch(0, [4, 5, 6]) == 2  # evicts 0 and 1, then stops
    assert not pool.resident(0, 0) and not pool.resident(0, 1)
    assert pool.resident(0, 2) and pool.resident(0, 3) and pool.resident(0, 4) and pool.resident(0, 5)
    assert not pool.resident(0, 6)
    pool.close()


def test_prefetched_experts_count_as_recent(moe):
    pool = make_pool(moe, 4)
    pool.prepare(0, np.array([[0, 1]], np.int32))
    pool.prefetch(0, [2, 3])
    pool.prepare(0, np.array([[4]], np.int32))  # evicts the least recent: 0, not the prefetched ones
    assert not pool.resident(0, 0) and pool.resident(0, 2) and pool.resident(0, 3)
    pool.close()


def test_usage_counts(moe):
    E, layers = 16, 3
    pool = make_pool(moe, 40, layers, E)
    rng = np.random.default_rng(4)
    ref = np.zeros((layers, E), np.uint64)
    for step in range(200):
        L = int(rng.integers(layers))
        ids = rng.integers(0, E, size=(2, 3)).astype(np.int32)
        ids[ids == 7] = -1  # dropped slots are not requests
        for e in set(ids.ravel().tolist()) - {-1}:
            ref[L, e] += 1
        pool.prepare(L, ids)
    assert np.array_equal(pool.usage(), ref)
    pool.close()


def test_pin_hot_keeps_the_most_requested(moe, tmp_path):
    E, layers = 16, 2
    rng = np.random.default_rng(8)
    p = 1.0 / np.arange(1, E + 1) ** 1.2
    p /= p.sum()
    trace = [(t % layers, rng.choice(E, size=(1, 3), replace=False, p=p).astype(np.int32)) for t in range(300)]
    first = make_pool(moe, 10, layers, E)
    for L, ids in trace:
        first.prepare(L, ids)
    counts = first.usage()
    first.save_usage(str(tmp_path / "usage.npy"))
    first.close()
    loaded = moe.MoePool.load_usage(str(tmp_path / "usage.npy"))
    assert np.array_equal(loaded, counts)
    # a new process: pin the 4 most requested, then run a trace that evicts heavily
    pool = make_pool(moe, 7, layers, E)
    assert pool.pin_hot(4 * block(moe, 4), counts=loaded) == 4
    order = sorted(((int(c), L * E + e) for (L, e), c in np.ndenumerate(loaded) if c > 0), key=lambda v: (-v[0], v[1]))
    hot = [(i // E, i % E) for _, i in order[:4]]
    assert all(pool.resident(L, e) for L, e in hot)
    for L, ids in trace[::-1]:
        pool.prepare(L, ids)
        assert all(pool.resident(L2, e2) for L2, e2 in hot)
    with pytest.raises(moe.MoeError):
        pool.pin_hot(100 * block(moe, 4))  # beyond the capacity
    pool.close()


def test_bookkeeping_pool_has_no_device_tables(moe):
    """A pool without a context keeps no device tables: asking for a layer's
    own table is an error, and prepare takes no table pointers; the widths of
    the latest call are still reported."""
    pool = moe.MoePool(None, 4 * moe.moe_expert_block_layout(4, 256, 128)[0], 2, 4, 256, 128)
    for e in range(4):
        pool.register(0, e, 4 if e % 2 else 2, None)
    with pytest.raises(moe.MoeError):
        pool.layer_table(0)
    pool.prepare(0, np.array([[1, 3]], np.int32))
    assert pool.call_widths() == 1 << 4
    pool.prepare(0, np.array([[0, 1]], np.int32))
    assert pool.call_widths() == (1 << 4) | (1 << 2)
    pool.prepare(0, np.array([[-1, -1]], np.int32))
    assert pool.call_widths() == 0
    assert pool.table_stats() == {"copies": 0, "skipped": 0}
    pool.close()
