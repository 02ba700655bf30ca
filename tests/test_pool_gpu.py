"""Expert pool on the GPU, through the C ABI: refilled slots hold exactly the
host blocks, and expert FFN outputs computed from pool tables are bit-equal
to those from an all-resident table, over many calls enqueued without
synchronisation while the pool keeps evicting (so every refill into memory
an earlier call still reads must wait for it), for one width and for a
mixed int4/int2 layer. Every slot a pool-backed call computes is also
compared directly with the oracle (its own packing of the same fp32 weights
and its own quantisation of the same hidden states), bit for bit.
"""
import numpy as np
import pytest

from tests.gpu_util import log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

H, I = 256, 128


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import quantized_moe_expert_sigmoid_amd as m
    m.lib()
    return m


@pytest.fixture(scope="module")
def ctx(moe):
    c = moe.MoeCtx(0)
    yield c
    c.close()


_hip = None


def dev_bytes(ptr, n):
    """Copy n bytes at a raw device address to a host uint8 tensor (hipMemcpy)."""
    import ctypes
    global _hip
    if _hip is None:
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    out = torch.empty(n, dtype=torch.uint8)
    assert _hip.hipMemcpy(out.data_ptr(), ptr, n, 2) == 0  # hipMemcpyDeviceToHost
    return out


def make_blocks(moe, ctx, syn, bits, E, seed):
    blocks = moe.ExpertBlocks(E, bits, H, I)
    for e in range(E):
        g, u, d = syn.expert_weights(seed, 0, e, H, I)
        blocks.pack_from_fp32(ctx, e, *(torch.from_numpy(a).cuda() for a in (g, u, d)))
    torch.cuda.synchronize()
    host = []
    for e in range(E):
        h = torch.empty(blocks.block_bytes, dtype=torch.uint8, pin_memory=True)
        h.copy_(blocks.data[e])
        host.append(h)
    return blocks, host


class OracleBlocks:
    """The oracle's own packing of the fp32 weights make_blocks packs on the
    GPU (same seeds), built lazily per (width, expert)."""

    def __init__(self, orc, syn, seed):
        self.orc, self.syn, self.seed, self.cache = orc, syn, seed, {}

    def get(self, bits, e):
        if (bits, e) not in self.cache:
            self.cache[(bits, e)] = self.orc.pack_expert(bits, *self.syn.expert_weights(self.seed, 0, e, H, I))
        return self.cache[(bits, e)]


def check_slots_vs_oracle(orc, syn, seed, y, ids, expert_of, shared_ex=None):
    """Every slot (t, j) of y against the oracle: expert_of(e) gives the
    oracle-packed expert (None: the slot was not computed here); slot k
    against shared_ex when given. Tokens are syn.hidden(seed, T, H),
    quantised by the oracle."""
    T, k = ids.shape
    xq, sx = orc.quantize_act(syn.hidden(seed, T, H))
    yh = y.cpu().numpy()
    n = 0
    for t in range(T):
        for j in range(k):
            ex = expert_of(int(ids[t, j]))
            if ex is None:
                continue
            r = orc.expert_token(ex, xq[t], float(sx[t]))["y"]
            assert np.array_equal(yh[t, j].view(np.uint32), r.view(np.uint32)), (t, j)
            n += 1
        if shared_ex is not None:
            r = orc.expert_token(shared_ex, xq[t], float(sx[t]))["y"]
            assert np.array_equal(yh[t, k].view(np.uint32), r.view(np.uint32)), t
            n += 1
    return n


def token_inputs(moe, ctx, syn, T, seed):
    x = torch.from_numpy(syn.hidden(seed, T, H)).cuda()
    xq = torch.empty((T, H), dtype=torch.int8, device="cuda")
    sx = torch.empty((T,), dtype=torch.float32, device="cuda")
    moe.moe_quantize_act_i8(ctx, x, xq, sx)
    return xq, sx


def test_refilled_slots_equal_host_blocks(moe, ctx, syn):
    E = 6
    blocks, host = make_blocks(moe, ctx, syn, 4, E, seed=31)
    pool = moe.MoePool(ctx, 3 * blocks.block_bytes, 1, E, H, I)
    for e in range(E):
        pool.register(0, e, 4, host[e])
    table = torch.zeros((E, 6), dtype=torch.int64, device="cuda")
    bits = torch.zeros((E,), dtype=torch.uint8, device="cuda")
    for ids in ([[0, 1]], [[2, 3]], [[1, 4]], [[5, 0]]):
        pool.prepare(0, np.array(ids, np.int32), table, bits)
        torch.cuda.synchronize()
        tab = table.cpu().numpy()
        bb = bits.cpu().numpy()
        for e in range(E):
            if pool.resident(0, e):
                assert bb[e] == 4
                got = dev_bytes(int(tab[e, 0]), blocks.block_bytes)
                assert torch.equal(got, host[e]), e
                # the table's six pointers follow the block layout
                assert [int(tab[e, j]) - int(tab[e, 0]) for j in range(6)] == blocks.offsets
            else:
                assert bb[e] == 0 and not tab[e].any()
    st = pool.stats()
    assert st["misses"] == 7 and st["hits"] == 1 and st["bytes_h2d"] == 7 * blocks.block_bytes
    pool.close()


@pytest.mark.parametrize("slots", [4, 8])
def test_pool_ffn_bit_equal_under_eviction(moe, ctx, orc, syn, slots):
    """40 calls, two tokens of top-2 each, enqueued back to back; the pool
    holds `slots` blocks (4 = one call's worst case, so calls keep evicting
    what the previous call read)."""
    E, T, k = 10, 2, 2
    blocks, host = make_blocks(moe, ctx, syn, 4, E, seed=32)
    shared_blocks, _ = make_blocks(moe, ctx, syn, 4, 1, seed=33)
    shared = shared_blocks.struct(0)
    pool = moe.MoePool(ctx, slots * blocks.block_bytes, 1, E, H, I)
    for e in range(E):
        pool.register(0, e, 4, host[e])
    table = torch.zeros((E, 6), dtype=torch.int64, device="cuda")
    bits = torch.zeros((E,), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(slots)
    calls = []
    for c in range(40):
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        xq, sx = token_inputs(moe, ctx, syn, T, seed=100 + c)
        idx = torch.from_numpy(ids).cuda()
        y = torch.zeros((T, k + 1, H), dtype=torch.float32, device="cuda")
        pool.prepare(0, ids, table, bits)
        moe.moe_expert_ffn_q4(ctx, table, shared, bits, xq, sx, idx, H, I, E, y)
        calls.append((xq, sx, idx, y))
    torch.cuda.synchronize()
    ctx.check()
    oe, osh = OracleBlocks(orc, syn, 32), OracleBlocks(orc, syn, 33).get(4, 0)
    for c, (xq, sx, idx, y) in enumerate(calls):
        ref = torch.zeros_like(y)
        moe.moe_expert_ffn_q4(ctx, blocks.table, shared, None, xq, sx, idx, H, I, E, ref)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), c
        check_slots_vs_oracle(orc, syn, 100 + c, y, idx.cpu().numpy(), lambda e: oe.get(4, e), osh)
    st = pool.stats()
    log(f"pool slots={slots}: {st}")
    assert st["hits"] + st["misses"] == sum(len(set(i.cpu().numpy().ravel())) for _, _, i, _ in calls)
    if slots == 4:
        assert st["misses"] > 60
    pool.close()


def test_pool_mixed_widths(moe, ctx, orc, syn):
    """Even experts int4, odd experts int2, two layers sharing one slab; one
    FFN call per width with the pool's width table."""
    E, T, k, L = 8, 3, 2, 2
    b4, h4 = make_blocks(moe, ctx, syn, 4, E, seed=34)
    b2, h2 = make_blocks(moe, ctx, syn, 2, E, seed=35)
    cap = 3 * b4.block_bytes + 3 * b2.block_bytes
    pool = moe.MoePool(ctx, cap, L, E, H, I)
    for layer in range(L):
        for e in range(E):
            if e % 2 == 0:
                pool.register(layer, e, 4, h4[e])
            else:
                pool.register(layer, e, 2, h2[e])
    ref_table = torch.stack([b4.table[e] if e % 2 == 0 else b2.table[e] for e in range(E)]).contiguous()
    ref_bits = torch.tensor([4 if e % 2 == 0 else 2 for e in range(E)], dtype=torch.uint8, device="cuda")
    table = torch.zeros((E, 6), dtype=torch.int64, device="cuda")
    bits = torch.zeros((E,), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(9)
    outs = []
    for c in range(24):
        layer = c % L
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        if len(set(ids.ravel()) & set(range(0, E, 2))) > 3 or len(set(ids.ravel()) & set(range(1, E, 2))) > 3:
            continue  # more of one width than the slab holds beside the other
        xq, sx = token_inputs(moe, ctx, syn, T, seed=200 + c)
        idx = torch.from_numpy(ids).cuda()
        y = torch.zeros((T, k + 1, H), dtype=torch.float32, device="cuda")
        try:
            pool.prepare(layer, ids, table, bits)
        except moe.MoeError as ex:  # first-fit fragmentation can refuse a mixed call
            assert ex.status == moe.MOE_EPOOL
            continue
        moe.moe_expert_ffn_q4(ctx, table, None, bits, xq, sx, idx, H, I, E, y)
        moe.moe_expert_ffn_q2(ctx, table, None, bits, xq, sx, idx, H, I, E, y)
        outs.append((c, xq, sx, idx, y))
    torch.cuda.synchronize()
    ctx.check()
    assert len(outs) >= 8
    o4, o2 = OracleBlocks(orc, syn, 34), OracleBlocks(orc, syn, 35)
    for c, xq, sx, idx, y in outs:
        ref = torch.zeros_like(y)
        moe.moe_expert_ffn_q4(ctx, ref_table, None, ref_bits, xq, sx, idx, H, I, E, ref)
        moe.moe_expert_ffn_q2(ctx, ref_table, None, ref_bits, xq, sx, idx, H, I, E, ref)
        torch.cuda.synchronize()
        assert torch.equal(y, ref)
        check_slots_vs_oracle(orc, syn, 200 + c, y, idx.cpu().numpy(),
                              lambda e: o4.get(4, e) if e % 2 == 0 else o2.get(2, e))
    pool.close()


def test_pool_capacity_refusal_and_reuse(moe, ctx, syn):
    E = 4
    blocks, host = make_blocks(moe, ctx, syn, 4, E, seed=36)
    pool = moe.MoePool(ctx, 2 * blocks.block_bytes, 1, E, H, I)
    for e in range(E):
        pool.register(0, e, 4, host[e], pin=(e == 0))
    table = torch.zeros((E, 6), dtype=torch.int64, device="cuda")
    pool.prepare(0, np.array([[0, 1]], np.int32), table)
    with pytest.raises(moe.MoeError) as ex:
        pool.prepare(0, np.array([[2, 3]], np.int32), table)  # expert 0 is pinned: one free block only
    assert ex.value.status == moe.MOE_EPOOL
    pool.prepare(0, np.array([[2]], np.int32), table)
    torch.cuda.synchronize()
    assert pool.resident(0, 0) and pool.resident(0, 2)
    tab = table.cpu().numpy()
    assert torch.equal(dev_bytes(int(tab[2, 0]), blocks.block_bytes), host[2])
    pool.close()


def test_pool_prefetch_bit_equal(moe, ctx, orc, syn):
    """Each call prefetches the next call's experts before its own FFN is
    enqueued (the prefetch may not evict what this call reads); outputs equal
    those from an all-resident table, and prefetched experts are hits."""
    E, T, k, slots = 10, 2, 2, 6
    blocks, host = make_blocks(moe, ctx, syn, 4, E, seed=37)
    pool = moe.MoePool(ctx, slots * blocks.block_bytes, 1, E, H, I)
    for e in range(E):
        pool.register(0, e, 4, host[e])
    table = torch.zeros((E, 6), dtype=torch.int64, device="cuda")
    bits = torch.zeros((E,), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(21)
    ids_all = [np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32) for _ in range(41)]
    calls = []
    for c in range(40):
        xq, sx = token_inputs(moe, ctx, syn, T, seed=300 + c)
        idx = torch.from_numpy(ids_all[c]).cuda()
        y = torch.zeros((T, k + 1, H), dtype=torch.float32, device="cuda")
        pool.prepare(0, ids_all[c], table, bits)
        pool.prefetch(0, ids_all[c + 1].ravel())
        moe.moe_expert_ffn_q4(ctx, table, None, bits, xq, sx, idx, H, I, E, y)
        calls.append((xq, sx, idx, y))
    torch.cuda.synchronize()
    ctx.check()
    oe = OracleBlocks(orc, syn, 37)
    for c, (xq, sx, idx, y) in enumerate(calls):
        ref = torch.zeros_like(y)
        moe.moe_expert_ffn_q4(ctx, blocks.table, None, None, xq, sx, idx, H, I, E, ref)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), c
        check_slots_vs_oracle(orc, syn, 300 + c, y, idx.cpu().numpy(), lambda e: oe.get(4, e))
    ps = pool.prefetch_stats()
    log(f"prefetch: {ps}, {pool.stats()}")
    assert ps["issued"] > 20 and ps["used"] > 10
    pool.close()


def test_pool_tiers_bit_equal(moe, ctx, orc, syn):
    """Precision tiers: three experts int8 with an int4 block, the others int4
    with an int2 block, demotion on, a slab under pressure; midway the hot
    experts are pinned (demoted copies re-loaded at full width). Every call's
    outputs equal those of an all-resident table at the widths the pool
    reported for that call, one FFN call per width."""
    E, T, k = 10, 2, 2
    b8, h8 = make_blocks(moe, ctx, syn, 8, E, seed=38)
    b4, h4 = make_blocks(moe, ctx, syn, 4, E, seed=38)
    b2, h2 = make_blocks(moe, ctx, syn, 2, E, seed=38)
    full = {e: (8 if e < 3 else 4) for e in range(E)}
    pool = moe.MoePool(ctx, 6 * b4.block_bytes, 1, E, H, I)
    for e in range(E):
        if full[e] == 8:
            pool.register(0, e, 8, h8[e])
            pool.register_alt(0, e, 4, h4[e])
        else:
            pool.register(0, e, 4, h4[e])
            pool.register_alt(0, e, 2, h2[e])
    pool.set_demotion(True)
    per_width = {8: b8, 4: b4, 2: b2}
    table = torch.zeros((E, 6), dtype=torch.int64, device="cuda")
    bits = torch.zeros((E,), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(23)
    calls = []
    for c in range(48):
        if c == 24:
            counts = np.zeros((1, E), np.uint64)
            counts[0, 0] = 9  # pin expert 0 (int8)
            assert pool.pin_hot(b8.block_bytes, counts) == 1
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        xq, sx = token_inputs(moe, ctx, syn, T, seed=400 + c)
        idx = torch.from_numpy(ids).cuda()
        y = torch.zeros((T, k + 1, H), dtype=torch.float32, device="cuda")
        try:
            pool.prepare(0, ids, table, bits)
        except moe.MoeError as ex:  # first-fit fragmentation can refuse a call
            assert ex.status == moe.MOE_EPOOL
            continue
        widths = {int(e): pool.resident_bits(0, int(e)) for e in set(ids.ravel())}
        for b in (8, 4, 2):
            getattr(moe, f"moe_expert_ffn_q{b}")(ctx, table, None, bits, xq, sx, idx, H, I, E, y)
        calls.append((c, xq, sx, idx, y, widths))
    torch.cuda.synchronize()
    ctx.check()
    ts = pool.tier_stats()
    log(f"tiers: {ts}, {pool.stats()}")
    assert len(calls) >= 40 and ts["demoted_loads"] > 5
    assert any(w < full[e] for *_, ws in calls for e, w in ws.items())
    ot = OracleBlocks(orc, syn, 38)
    for c, xq, sx, idx, y, widths in calls:
        wv = [widths.get(e, 0) for e in range(E)]
        ref_table = torch.stack([per_width[w].table[e] if w else b4.table[e] for e, w in enumerate(wv)]).contiguous()
        ref_bits = torch.tensor(wv, dtype=torch.uint8, device="cuda")
        ref = torch.zeros_like(y)
        for b in (8, 4, 2):
            getattr(moe, f"moe_expert_ffn_q{b}")(ctx, ref_table, None, ref_bits, xq, sx, idx, H, I, E, ref)
        torch.cuda.synchronize()
        assert torch.equal(y, ref), (c, widths)
        check_slots_vs_oracle(orc, syn, 400 + c, y, idx.cpu().numpy(), lambda e: ot.get(widths[e], e))
        if c >= 24 and 0 in widths:  # pinned before call 24: full width from then on
            assert widths[0] == 8, (c, widths)
    pool.close()


def test_pool_table_and_widths_in_one_buffer(moe, ctx, syn):
    """When the widths start right after the table, prepare writes both with
    one copy; the contents equal those written into separate buffers."""
    E = 6
    b4, h4 = make_blocks(moe, ctx, syn, 4, E, seed=39)
    b2, h2 = make_blocks(moe, ctx, syn, 2, E, seed=39)
    pool = moe.MoePool(ctx, 3 * b4.block_bytes, 1, E, H, I)
    for e in range(E):
        pool.register(0, e, 4 if e % 2 == 0 else 2, h4[e] if e % 2 == 0 else h2[e])
    sep_t = torch.zeros((E, 6), dtype=torch.int64, device="cuda")
    sep_b = torch.zeros((E,), dtype=torch.uint8, device="cuda")
    one = torch.zeros((E * 48 + E,), dtype=torch.uint8, device="cuda")
    one_t, one_b = one[:E * 48].view(torch.int64).view(E, 6), one[E * 48:]
    for ids in ([[0, 1]], [[2, 3]], [[4, 1]]):
        pool.prepare(0, np.array(ids, np.int32), sep_t, sep_b)
        pool.prepare(0, np.array(ids, np.int32), one_t, one_b)  # all hits: the same residency
        torch.cuda.synchronize()
        assert torch.equal(sep_t, one_t) and torch.equal(sep_b, one_b)
        assert set(np.nonzero(one_b.cpu().numpy())[0]) >= set(np.array(ids).ravel())
    pool.close()


def test_pool_own_tables_copy_only_changes(moe, ctx, syn):
    """The pool's own per-layer tables: prepare copies a layer's table there
    only when its bytes changed since its last copy there. After every call
    the own table equals the table the same residency gives in a caller's
    buffer, and a copy is skipped exactly when the bytes equal the layer's
    previous ones (each call is made twice in a row: the repeat always
    skips). Pointers into another layer's own table are rejected."""
    E, L = 6, 2
    b4, h4 = make_blocks(moe, ctx, syn, 4, E, seed=41)
    b2, h2 = make_blocks(moe, ctx, syn, 2, E, seed=41)
    pool = moe.MoePool(ctx, 3 * b4.block_bytes, L, E, H, I)
    try:
        for layer in range(L):
            for e in range(E):
                pool.register(layer, e, 4 if e % 3 else 2, h4[e] if e % 3 else h2[e])
        own = [pool.layer_table(layer) for layer in range(L)]
        assert own[1][0] != own[0][0] and own[0][1] == own[0][0] + E * 48
        ext = torch.zeros((E * 48 + E,), dtype=torch.uint8, device="cuda")
        ext_t, ext_b = ext[:E * 48].view(torch.int64).view(E, 6), ext[E * 48:]
        rng = np.random.default_rng(5)
        last = [None] * L
        n_skip = n_copy = 0
        for step in range(30):
            layer = int(rng.integers(0, L))
            ids = rng.choice(E, size=2, replace=False).astype(np.int32)[None, :]
            for rep in range(2):
                c0 = pool.table_stats()
                pool.prepare(layer, ids, own[layer][0], own[layer][1])
                c1 = pool.table_stats()
                pool.prepare(layer, ids, ext_t, ext_b)  # all hits: the same residency
                torch.cuda.synchronize()
                want = ext.cpu()
                got = dev_bytes(own[layer][0], E * 48 + E)
                assert torch.equal(got, want), (step, rep)
                same = last[layer] is not None and torch.equal(want, last[layer])
                assert same or rep == 0, (step, rep)
                made = (c1["skipped"] - c0["skipped"], c1["copies"] - c0["copies"])
                assert made == ((1, 0) if same else (0, 1)), (step, rep)
                n_skip += int(same)
                n_copy += int(not same)
                last[layer] = want
        assert n_skip >= 30 and n_copy > 2
        with pytest.raises(moe.MoeError):
            pool.prepare(0, np.array([[0]], np.int32), own[1][0], own[1][1])
        with pytest.raises(moe.MoeError):
            pool.prepare(0, np.array([[0]], np.int32), own[0][0], ext_b)
        with pytest.raises(moe.MoeError):
            pool.prepare(0, np.array([[0]], np.int32), ext_t, own[1][1])
    finally:
        pool.close()


@pytest.mark.parametrize("slots", [8, 10])
def test_pool_one_token_mixed_loop(moe, ctx, orc, syn, slots):
    """The decode loop through the pool, one token per call, as the stack
    benchmark runs it: prepare into the layer's own table, the call's widths,
    one mixed-width FFN call with the combine. 40 calls over two layers are
    enqueued back to back while the pool keeps evicting (the two layers'
    blocks take about 13 int4-block sizes; 8 slots always leave room for a
    call's three experts whatever the first-fit placement left behind, as
    2 hits split at most 6 free slots into 3 extents); every call's slots
    and output equal those of the same mixed call on an all-resident table,
    and the output equals moe_combine over its slots."""
    E, k, L = 8, 3, 2
    b4, h4 = make_blocks(moe, ctx, syn, 4, E, seed=37)
    b2, h2 = make_blocks(moe, ctx, syn, 2, E, seed=37)
    shared_blocks, _ = make_blocks(moe, ctx, syn, 4, 1, seed=38)
    shared = shared_blocks.struct(0)
    wbits = np.array([4, 2, 4, 4, 2, 4, 2, 4], np.uint8)
    full = torch.where(torch.from_numpy(wbits == 4).cuda()[:, None], b4.table, b2.table).contiguous()
    full_bits = torch.from_numpy(wbits).cuda()
    pool = moe.MoePool(ctx, slots * b4.block_bytes, L, E, H, I)
    try:
        for layer in range(L):
            for e in range(E):
                pool.register(layer, e, int(wbits[e]), h4[e] if wbits[e] == 4 else h2[e])
        own = [pool.layer_table(layer) for layer in range(L)]
        rng = np.random.default_rng(slots)
        calls = []
        for c in range(40):
            layer = c % L
            ids = rng.choice(E, size=k, replace=False).astype(np.int32)[None, :]
            wts = torch.from_numpy(rng.random((1, k)).astype(np.float32)).cuda()
            xq, sx = token_inputs(moe, ctx, syn, 1, seed=200 + c)
            idx = torch.from_numpy(ids).cuda()
            y = torch.zeros((1, k + 1, H), dtype=torch.float32, device="cuda")
            out = torch.empty((1, H), dtype=torch.float32, device="cuda")
            pool.prepare(layer, ids, own[layer][0], own[layer][1])
            mask = pool.call_widths() | (1 << 4)
            assert mask == sum({1 << int(wbits[e]) for e in ids[0]} | {1 << 4})
            moe.moe_expert_ffn_mixed(ctx, own[layer][0], shared, 4, own[layer][1], mask, xq, sx, idx, H, I, E, y,
                                     topk_w=wts, out=out)
            calls.append((xq, sx, idx, wts, mask, y, out))
        torch.cuda.synchronize()
        ctx.check()
        assert pool.table_stats()["skipped"] > 0
        oe, osh = OracleBlocks(orc, syn, 37), OracleBlocks(orc, syn, 38).get(4, 0)
        for c, (xq, sx, idx, wts, mask, y, out) in enumerate(calls):
            check_slots_vs_oracle(orc, syn, 200 + c, y, idx.cpu().numpy(), lambda e: oe.get(int(wbits[e]), e), osh)
            ry = torch.zeros_like(y)
            ro = torch.empty_like(out)
            moe.moe_expert_ffn_mixed(ctx, full, shared, 4, full_bits, mask, xq, sx, idx, H, I, E, ry, topk_w=wts,
                                     out=ro)
            rc = torch.empty_like(out)
            moe.moe_combine(ctx, y, wts, True, rc)
            torch.cuda.synchronize()
            assert torch.equal(y, ry) and torch.equal(out, ro) and torch.equal(out, rc), c
    finally:
        pool.close()


def test_pool_stream_rebind(moe, orc, syn):
    """A context re-bound to another stream between calls: the pool makes the
    new stream wait for the refills of the experts it reads and copies the
    layer's own table again on it (a wait or a copy on the previous stream
    does not order the new stream's kernels). Calls come in pairs with the
    same experts, each pair on the other stream: the first call of a pair
    copies the table, the second (all hits, same stream) skips the copy.
    Every slot equals the same call on an all-resident table and the
    oracle's result, bit for bit."""
    E, k = 8, 2
    c2 = moe.MoeCtx(0)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    pool = None
    try:
        blocks, host = make_blocks(moe, c2, syn, 4, E, seed=39)
        pool = moe.MoePool(c2, 4 * blocks.block_bytes, 1, E, H, I)
        for e in range(E):
            pool.register(0, e, 4, host[e])
        tab, wid = pool.layer_table(0)
        rng = np.random.default_rng(39)
        calls = []
        for c in range(24):
            ids = rng.choice(E, size=k, replace=False).astype(np.int32)[None, :] if c % 2 == 0 else calls[-1][0]
            xq, sx = token_inputs(moe, c2, syn, 1, seed=300 + c)
            y = torch.zeros((1, k + 1, H), dtype=torch.float32, device="cuda")
            calls.append((ids, xq, sx, torch.from_numpy(ids).cuda(), y))
        torch.cuda.synchronize()
        for c, (ids, xq, sx, idx, y) in enumerate(calls):
            c2.set_stream(streams[(c // 2) % 2])
            t0 = pool.table_stats()
            pool.prepare(0, ids, tab, wid)
            t1 = pool.table_stats()
            made = (t1["copies"] - t0["copies"], t1["skipped"] - t0["skipped"])
            assert made == ((1, 0) if c % 2 == 0 else (0, 1)), (c, made)
            moe.moe_expert_ffn_mixed(c2, tab, None, 4, wid, 1 << 4, xq, sx, idx, H, I, E, y)
        c2.set_stream(torch.cuda.current_stream())
        torch.cuda.synchronize()
        c2.check()
        oe = OracleBlocks(orc, syn, 39)
        all4 = torch.full((E,), 4, dtype=torch.uint8, device="cuda")
        for c, (ids, xq, sx, idx, y) in enumerate(calls):
            ref = torch.zeros_like(y)
            moe.moe_expert_ffn_mixed(c2, blocks.table, None, 4, all4, 1 << 4, xq, sx, idx, H, I, E, ref)
            torch.cuda.synchronize()
            assert torch.equal(y, ref), c
            check_slots_vs_oracle(orc, syn, 300 + c, y, ids, lambda e: oe.get(4, e))
        st = pool.stats()
        log(f"pool stream rebind: {st}")
        assert st["misses"] > 8
    finally:
        if pool is not None:
            pool.close()
        c2.close()
