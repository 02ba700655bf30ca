"""GPU parity at sizes the oracle finishes in seconds (several tiles, ragged
tails), through the C ABI. Bar: bit-exact for packed weights, activation
codes and scales, integer accumulators, requantised intermediates and expert
outputs; router indices exact away from near-ties; combined outputs within
1e-3 of the per-row max (fp32 accumulation vs the oracle's fp64).
"""
import numpy as np
import pytest

from tests.gpu_util import compare_router, log, rel_row_err

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


# --------------------------------------------------------------------------
# quantisation
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [8, 4, 2])
@pytest.mark.parametrize("R,C", [(37, 320), (5, 64), (300, 6144)])
def test_quantize_rows_bitexact(moe, ctx, orc, syn, bits, R, C):
    log(f"quantize_rows bits={bits} R={R} C={C}")
    w = syn.normal(11, syn.stream_id(syn.K_MISC, R, C), (R, C), 0.02)
    w[R // 2] = 0.0
    ref_p, ref_s = orc.quantize_rows(bits, w)
    p = torch.empty((R, C * bits // 8), dtype=torch.uint8, device="cuda")
    s = torch.empty((R,), dtype=torch.float32, device="cuda")
    moe.moe_quantize_rows(ctx, bits, dev(w), p, s)
    assert np.array_equal(host(p), ref_p)
    assert np.array_equal(host(s).view(np.uint32), ref_s.view(np.uint32))


def test_quantize_rows_half_ties(moe, ctx, orc):
    # values exactly halfway between codes: round half to even on both sides
    w = np.tile(np.array([3.5, -1.75, 0.25, 0, 0.75, -3.5, 1.25, 0.5], np.float32), (4, 8))
    for bits in (8, 4, 2):
        ref_p, ref_s = orc.quantize_rows(bits, w)
        p = torch.empty((4, 64 * bits // 8), dtype=torch.uint8, device="cuda")
        s = torch.empty((4,), dtype=torch.float32, device="cuda")
        moe.moe_quantize_rows(ctx, bits, dev(w), p, s)
        assert np.array_equal(host(p), ref_p) and np.array_equal(host(s), ref_s)


@pytest.mark.parametrize("T,H", [(1, 6144), (33, 128), (64, 6144), (3, 8192), (5, 64), (4, 1088)])
def test_quantize_act_bitexact(moe, ctx, orc, syn, T, H):
    log(f"quantize_act T={T} H={H}")
    x = syn.hidden(21, T, H)
    if T > 2:
        x[1] = 0.0
    ref_q, ref_s = orc.quantize_act(x)
    q = torch.empty((T, H), dtype=torch.int8, device="cuda")
    s = torch.empty((T,), dtype=torch.float32, device="cuda")
    moe.moe_quantize_act_i8(ctx, dev(x), q, s)
    assert np.array_equal(host(q), ref_q)
    assert np.array_equal(host(s), ref_s)


# --------------------------------------------------------------------------
# router and bucketing
# --------------------------------------------------------------------------

def run_router(moe, ctx, x, wr, bias, k, logits_in=False, scale=1.0):
    T = x.shape[0]
    idx = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    moe.moe_router_topk(ctx, dev(x), None if wr is None else dev(wr), None if bias is None else dev(bias), k, idx, w,
                        scale, logits_in=logits_in)
    return host(idx), host(w)


@pytest.mark.parametrize("T,H,E,k", [(32, 128, 8, 2), (1, 6144, 256, 8), (7, 6144, 256, 8), (64, 6144, 256, 8),
                                     (130, 384, 64, 6), (5, 128, 8, 8)])
def test_router_hidden(moe, ctx, orc, syn, T, H, E, k):
    log(f"router T={T} H={H} E={E} k={k}")
    x = syn.hidden(31, T, H)
    wr = syn.router_weights(31, 0, E, H)
    bias = syn.router_bias(31, 0, E)
    idx_o, w_o, keys, sig = orc.router(x, wr, bias, k, want_keys=True)
    idx_g, w_g = run_router(moe, ctx, x, wr, bias, k)
    near = compare_router(idx_g, w_g, idx_o, keys, sig)
    assert near <= max(1, T // 50)


def test_router_logits_zipf_and_ties(moe, ctx, orc, syn):
    z = syn.zipf_logits(2, 0, 64, 256, 1.1)
    idx_o, w_o, keys, sig = orc.router(z, None, None, 8, logits_in=True, want_keys=True)
    idx_g, w_g = run_router(moe, ctx, z, None, None, 8, logits_in=True)
    compare_router(idx_g, w_g, idx_o, keys, sig)
    # exact ties: equal keys go to the lower expert id
    zt = np.array([[0.5, 1.0, 1.0, -2.0, 1.0, 0.5, 0.0, 0.0]], np.float32)
    idx_g, w_g = run_router(moe, ctx, zt, None, None, 4, logits_in=True)
    assert idx_g[0].tolist() == [1, 2, 4, 0]
    # routed scale multiplies the normalised weights
    idx_g, w_g = run_router(moe, ctx, zt, None, None, 2, logits_in=True, scale=2.5)
    assert abs(w_g[0].sum() - 2.5) < 1e-5


# above 4096 (token, slot) entries the bucketing runs in chunks of tokens
# (a count pass and a placement pass): 2048, 2049 (a last chunk of one
# token), 700 x 8, 1500 x 16 over 1024 experts, 10000 (160-token chunks)
@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (64, 256, 8), (2048, 256, 8), (37, 8, 2), (1500, 1024, 16),
                                   (2049, 256, 8), (700, 64, 8), (10000, 256, 8)])
def test_bucket_exact(moe, ctx, orc, syn, T, E, k):
    log(f"bucket T={T} E={E} k={k}")
    z = syn.normal(5, syn.stream_id(syn.K_MISC, T, E), (T, E))
    idx, _ = orc.router(z, None, None, k, logits_in=True)
    c_o, o_o, p_o = orc.bucket(idx, E)
    c = torch.empty((E,), dtype=torch.int32, device="cuda")
    o = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    p = torch.empty((T * k,), dtype=torch.int32, device="cuda")
    moe.moe_bucket_tokens(ctx, dev(idx), E, c, o, p)
    assert np.array_equal(host(c), c_o) and np.array_equal(host(o), o_o) and np.array_equal(host(p), p_o)


def test_bucket_bad_index_reported_chunked(moe, ctx, orc, syn):
    """An id out of range in a call large enough for the chunked bucketing:
    the flag is raised and the other entries are counted and placed as the
    oracle does without the bad one."""
    T, E, k = 1024, 64, 8
    z = syn.normal(6, syn.stream_id(syn.K_MISC, T, E), (T, E))
    idx, _ = orc.router(z, None, None, k, logits_in=True)
    idx = idx.copy()
    idx[700, 3] = E + 5
    # expected: every other entry, each expert's in ascending (token, slot)
    # order (a stable sort of the flat entries by expert; the bad one last)
    flat = idx.ravel()
    key = np.where(flat < E, flat, E)
    c_o = np.bincount(flat[flat < E], minlength=E).astype(np.int32)
    o_o = np.concatenate([[0], np.cumsum(c_o)]).astype(np.int32)
    p_o = np.argsort(key, kind="stable").astype(np.int32)
    c = torch.empty((E,), dtype=torch.int32, device="cuda")
    o = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    p = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
    moe.moe_bucket_tokens(ctx, dev(idx), E, c, o, p)
    with pytest.raises(moe.MoeError):
        ctx.check()
    ctx.check()  # cleared
    n = int(o_o[-1])
    assert np.array_equal(host(c), c_o) and np.array_equal(host(o), o_o) and np.array_equal(host(p)[:n], p_o[:n])


@pytest.mark.parametrize("T", [100, 1024])
def test_bucket_dropped_slots(moe, ctx, orc, syn, T):
    """Ids of -1 (slots dropped by top-p) name no expert: they get no entry and
    raise no error, in the one-workgroup bucketing (T = 100) and in the chunked
    one (T = 1024, 8192 entries). Expected: a stable sort of the other entries by
    expert, so each expert's list is in (token, slot) order."""
    E, k = 64, 8
    z = syn.normal(7, syn.stream_id(syn.K_MISC, T, E), (T, E))
    idx, _ = orc.router(z, None, None, k, logits_in=True)
    idx = idx.copy()
    rng = np.random.default_rng(T)
    drop = rng.random(idx.shape) < 0.15
    drop[:, 0] = False  # top-p keeps at least the first slot
    idx[drop] = -1
    flat = idx.ravel()
    c_o = np.bincount(flat[flat >= 0], minlength=E).astype(np.int32)
    o_o = np.concatenate([[0], np.cumsum(c_o)]).astype(np.int32)
    p_o = np.argsort(np.where(flat >= 0, flat, E), kind="stable").astype(np.int32)[: int(o_o[-1])]
    c = torch.empty((E,), dtype=torch.int32, device="cuda")
    o = torch.empty((E + 1,), dtype=torch.int32, device="cuda")
    p = torch.full((T * k,), -1, dtype=torch.int32, device="cuda")
    moe.moe_bucket_tokens(ctx, dev(idx), E, c, o, p)
    ctx.check()
    assert np.array_equal(host(c), c_o) and np.array_equal(host(o), o_o)
    assert np.array_equal(host(p)[: int(o_o[-1])], p_o)


def test_bucket_bad_index_reported(moe, ctx):
    idx = torch.tensor([[0, 9], [1, 2]], dtype=torch.int32, device="cuda")
    c = torch.empty((8,), dtype=torch.int32, device="cuda")
    o = torch.empty((9,), dtype=torch.int32, device="cuda")
    p = torch.full((4,), -1, dtype=torch.int32, device="cuda")
    moe.moe_bucket_tokens(ctx, idx, 8, c, o, p)
    with pytest.raises(moe.MoeError):
        ctx.check()
    assert host(c).sum() == 3
    ctx.check()  # cleared


def test_invalid_arguments_rejected(moe, ctx):
    x = torch.zeros((2, 100), dtype=torch.float32, device="cuda")  # H not a multiple of 64
    with pytest.raises(moe.MoeError):
        moe.moe_quantize_act_i8(ctx, x, torch.empty((2, 100), dtype=torch.int8, device="cuda"),
                                torch.empty((2,), dtype=torch.float32, device="cuda"))
    # T = 0 is a no-op
    moe.moe_quantize_act_i8(ctx, torch.zeros((0, 64), device="cuda"), torch.empty((0, 64), dtype=torch.int8,
                            device="cuda"), torch.empty((0,), device="cuda"))


# --------------------------------------------------------------------------
# expert FFN stage with captured intermediates
# --------------------------------------------------------------------------

def make_experts(moe, orc, syn, bits, H, I, E, seed):
    """GPU expert blocks packed on the GPU and the oracle's own packing of the
    same fp32 weights (never the GPU's bytes)."""
    blocks = moe.ExpertBlocks(E, bits, H, I)
    shared = moe.ExpertBlocks(1, bits, H, I)
    ctx = moe.MoeCtx(0)
    oexp = []
    for e in range(E):
        wg, wu, wd = syn.expert_weights(seed, 0, e, H, I)
        blocks.pack_from_fp32(ctx, e, dev(wg), dev(wu), dev(wd))
        oexp.append(orc.pack_expert(bits, wg, wu, wd))
    wg, wu, wd = syn.expert_weights(seed, 0, 0, H, I, shared=True)
    shared.pack_from_fp32(ctx, 0, dev(wg), dev(wu), dev(wd))
    osh = orc.pack_expert(bits, wg, wu, wd)
    torch.cuda.synchronize()
    ctx.close()
    return blocks, shared, oexp, osh


def random_routing(syn, T, E, k, seed):
    z = syn.normal(seed, syn.stream_id(syn.K_MISC, 77, T), (T, E))
    return np.argsort(-z, axis=1, kind="stable")[:, :k].astype(np.int32)


def check_ffn_intermediates(moe, ctx, orc, syn, kern, bits, T, H, I, E, k, idx, seed, with_shared=True):
    """Every intermediate of every (token, slot) pair bit-equal to the oracle's
    (slots of id -1, and the shared slot without a shared expert, untouched)."""
    log(f"ffn kernels={kern} bits={bits} T={T} H={H} I={I} E={E} k={k} shared={with_shared}")
    blocks, shared, oexp, osh = make_experts(moe, orc, syn, bits, H, I, E, seed=seed)
    x = syn.hidden(seed + 1, T, H)
    xq_o, sx_o = orc.quantize_act(x)
    P = T * (k + 1)
    dbg = dict(accg=torch.zeros((P, I), dtype=torch.int32, device="cuda"),
               accu=torch.zeros((P, I), dtype=torch.int32, device="cuda"),
               a=torch.zeros((P, I), dtype=torch.float32, device="cuda"),
               aq=torch.zeros((P, I), dtype=torch.int8, device="cuda"),
               sa=torch.zeros((P,), dtype=torch.float32, device="cuda"),
               accd=torch.zeros((P, H), dtype=torch.int32, device="cuda"))
    y = torch.full((T, k + 1, H), 7.0, dtype=torch.float32, device="cuda")
    ctx.set_debug(dbg)
    ctx.set_ffn_kernels(kern)
    try:
        sh = shared.struct(0) if with_shared else None
        moe.FFN_BY_BITS[bits](ctx, blocks.table, sh, None, dev(xq_o), dev(sx_o), dev(idx), H, I, E, y)
        ctx.check()
    finally:
        ctx.set_debug(None)
        ctx.set_ffn_kernels("auto")
    got = {n: host(t) for n, t in dbg.items()}
    yg = host(y)
    for t in range(T):
        for j in range(k + 1):
            if (j == k and not with_shared) or (j < k and idx[t, j] == -1):
                assert np.all(yg[t, j] == 7.0) and not got["accg"][t * (k + 1) + j].any(), (t, j)
                continue
            ex = osh if j == k else oexp[idx[t, j]]
            r = orc.expert_token(ex, xq_o[t], float(sx_o[t]))
            p = t * (k + 1) + j
            assert np.array_equal(got["accg"][p], r["accg"]), (t, j)
            assert np.array_equal(got["accu"][p], r["accu"]), (t, j)
            assert np.array_equal(got["a"][p].view(np.uint32), r["a"].view(np.uint32)), (t, j)
            assert np.array_equal(got["aq"][p], r["aq"]), (t, j)
            assert got["sa"][p] == np.float32(r["sa"]), (t, j)
            assert np.array_equal(got["accd"][p], r["accd"]), (t, j)
            assert np.array_equal(yg[t, j].view(np.uint32), r["y"].view(np.uint32)), (t, j)


@pytest.mark.parametrize("kern", ["dot4", "mfma", "auto"])
@pytest.mark.parametrize("bits", [4, 8, 2])
@pytest.mark.parametrize("T,H,I,E,k", [(32, 128, 64, 8, 2), (37, 256, 192, 8, 2), (3, 512, 128, 16, 4),
                                       (150, 256, 128, 4, 2), (2, 256, 128, 8, 3), (4, 128, 64, 6, 2)])
def test_ffn_intermediates_bitexact(moe, ctx, orc, syn, kern, bits, T, H, I, E, k):
    """Every intermediate of every (token, slot) pair bit-exact, for each
    kernel family ("auto": up to 3 tokens the single-token kernels once per
    token, more the matrix cores)."""
    idx = random_routing(syn, T, E, k, 42)
    check_ffn_intermediates(moe, ctx, orc, syn, kern, bits, T, H, I, E, k, idx, seed=40 + bits)


@pytest.mark.parametrize("bits", [4, 8, 2])
@pytest.mark.parametrize("H,I,E,k,shared", [(128, 64, 8, 2, True), (512, 192, 16, 8, True), (256, 128, 8, 3, False),
                                            (1024, 448, 40, 6, False), (64, 64, 2, 1, True), (128, 64, 4, 4, False),
                                            (8192, 128, 8, 2, True)])
def test_ffn_one_token(moe, ctx, orc, syn, bits, H, I, E, k, shared):
    """One token through the per-step expert FFN: the single-token kernels with
    the routing given (the default for T = 1; hidden 8192 is past their limit
    and takes the vector kernels) and the vector kernels, every intermediate
    bit-exact against the oracle; then a token with dropped slots (id -1),
    whose slots stay untouched."""
    idx = random_routing(syn, 1, E, k, 90 + k)
    for kern in ("auto", "dot4"):
        check_ffn_intermediates(moe, ctx, orc, syn, kern, bits, 1, H, I, E, k, idx, seed=91 + bits, with_shared=shared)
    idx[0, 1:k:2] = -1
    check_ffn_intermediates(moe, ctx, orc, syn, "auto", bits, 1, H, I, E, k, idx, seed=91 + bits, with_shared=shared)


def test_ffn_one_token_nothing_to_do(moe, ctx, orc, syn):
    """A token whose slots are all -1 (or of another width) and no shared
    expert: the call writes nothing."""
    H, I, E, k = 256, 128, 8, 3
    blocks, _, _, _ = make_experts(moe, orc, syn, 4, H, I, E, seed=95)
    xq_o, sx_o = orc.quantize_act(syn.hidden(96, 1, H))
    y = torch.full((1, k + 1, H), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn_q4(ctx, blocks.table, None, None, dev(xq_o), dev(sx_o), dev(np.full((1, k), -1, np.int32)),
                          H, I, E, y)
    eb = dev(np.full(E, 2, np.uint8))
    moe.moe_expert_ffn_q4(ctx, blocks.table, None, eb, dev(xq_o), dev(sx_o), dev(np.array([[0, 3, 5]], np.int32)),
                          H, I, E, y)
    ctx.check()
    assert np.all(host(y) == 7.0)


@pytest.mark.parametrize("T", [1, 4])
def test_ffn_repeated_and_bad_ids(moe, ctx, orc, syn, T):
    """An id repeated within a token, or outside [0, E), is reported by the
    context check; the slots with valid first ids are still computed and the
    offending slots are left untouched."""
    H, I, E, k = 256, 128, 8, 3
    blocks, shared, oexp, osh = make_experts(moe, orc, syn, 4, H, I, E, seed=97)
    xq_o, sx_o = orc.quantize_act(syn.hidden(98, T, H))
    for bad, ok in (([2, 5, 2], [0, 1]), ([2, 9, 5], [0, 2]), ([-3, 5, 1], [1, 2]), ([4, 4, 4], [0])):
        idx = np.repeat(np.array([bad], np.int32), T, axis=0)
        y = torch.full((T, k + 1, H), 7.0, dtype=torch.float32, device="cuda")
        moe.moe_expert_ffn_q4(ctx, blocks.table, shared.struct(0), None, dev(xq_o), dev(sx_o), dev(idx), H, I, E, y)
        with pytest.raises(moe.MoeError):
            ctx.check()
        yg = host(y)
        for t in range(T):
            for j in range(k):
                if j in ok:
                    r = orc.expert_token(oexp[idx[t, j]], xq_o[t], float(sx_o[t]))
                    assert np.array_equal(yg[t, j], r["y"]), (bad, t, j)
                else:
                    assert np.all(yg[t, j] == 7.0), (bad, t, j)
            assert np.array_equal(yg[t, k], orc.expert_token(osh, xq_o[t], float(sx_o[t]))["y"])


@pytest.mark.parametrize("E", [64, 14])
@pytest.mark.parametrize("bits", [4, 8, 2])
def test_ffn_mfma_tile_boundaries(moe, ctx, orc, syn, bits, E):
    """Per-expert token counts on both sides of every tile boundary of the
    matrix-core kernels (tiles of 64 tokens): 16, 17, 64, 65, 80, 81, 128, 129,
    144, 145, 256, 257, 1 and 0 tokens (145 = two full tiles and a third of
    17, 257 = four and one of 1); the shared expert takes all 1383 (21 full
    tiles and a remainder of 39). With 64 experts (50 of them unused: few
    tokens per expert on average) a remainder of up to 16 tokens is a
    one-block tile; with 14 (many per expert) every remainder is a full-size
    tile beside the expert's other tiles."""
    counts = [16, 17, 64, 65, 80, 81, 128, 129, 144, 145, 256, 257, 1, 0]
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    rng = np.random.default_rng(7)
    idx = rng.permutation(ids).reshape(-1, 1).astype(np.int32)
    check_ffn_intermediates(moe, ctx, orc, syn, "mfma", bits, idx.shape[0], 128, 64, E, 1, idx,
                            seed=45 + bits)


def test_ffn_kernel_selector_rejects_unknown_values(moe, ctx):
    for bad in (-1, 3, 7):
        with pytest.raises(moe.MoeError) as ex:
            ctx.set_ffn_kernels(bad)
        assert ex.value.status == moe.MOE_EINVAL
    ctx.set_ffn_kernels("auto")


def test_ffn_without_shared_leaves_slot(moe, ctx, orc, syn):
    H, I, E, k, T = 128, 64, 8, 2, 5
    blocks, shared, oexp, osh = make_experts(moe, orc, syn, 4, H, I, E, seed=50)
    x = syn.hidden(51, T, H)
    xq_o, sx_o = orc.quantize_act(x)
    idx = random_routing(syn, T, E, k, 52)
    y = torch.full((T, k + 1, H), 7.0, dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn_q4(ctx, blocks.table, None, None, dev(xq_o), dev(sx_o), dev(idx), H, I, E, y)
    yg = host(y)
    assert np.all(yg[:, k] == 7.0)
    for t in range(T):
        r = orc.expert_token(oexp[idx[t, 0]], xq_o[t], float(sx_o[t]))
        assert np.array_equal(yg[t, 0], r["y"])


@pytest.mark.parametrize("T", [9, 1])
def test_ffn_mixed_precision_filter(moe, ctx, orc, syn, T):
    """expert_bits selects which experts a width's entry point computes: a
    mixed int4/int2 layer is two calls writing disjoint slots (one token: the
    single-token kernels, several: the matrix-core kernels)."""
    H, I, E, k = 256, 128, 8, 3
    b4, sh4, o4, osh4 = make_experts(moe, orc, syn, 4, H, I, E, seed=60)
    b2, _, o2, _ = make_experts(moe, orc, syn, 2, H, I, E, seed=60)
    bits = np.array([4, 2, 4, 2, 2, 4, 4, 2], np.uint8)
    # one table: int4 blocks for 4-bit experts, int2 blocks for the others
    table = torch.where(torch.from_numpy(bits == 4).cuda()[:, None], b4.table, b2.table).contiguous()
    x = syn.hidden(61, T, H)
    xq_o, sx_o = orc.quantize_act(x)
    idx = random_routing(syn, T, E, k, 62)
    y = torch.zeros((T, k + 1, H), dtype=torch.float32, device="cuda")
    eb = dev(bits)
    moe.moe_expert_ffn_q4(ctx, table, sh4.struct(0), eb, dev(xq_o), dev(sx_o), dev(idx), H, I, E, y)
    moe.moe_expert_ffn_q2(ctx, table, None, eb, dev(xq_o), dev(sx_o), dev(idx), H, I, E, y)
    yg = host(y)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            ex = o4[e] if bits[e] == 4 else o2[e]
            assert np.array_equal(yg[t, j], orc.expert_token(ex, xq_o[t], float(sx_o[t]))["y"]), (t, j)
        assert np.array_equal(yg[t, k], orc.expert_token(osh4, xq_o[t], float(sx_o[t]))["y"])


@pytest.mark.parametrize("T", [1, 6])
@pytest.mark.parametrize("shared_bits", [4, 8, None])
def test_ffn_mixed_one_call(moe, ctx, orc, syn, T, shared_bits):
    """moe_expert_ffn_mixed: a layer of int8, int4 and int2 experts in one
    call, every slot bit-exact against the oracle at its expert's width (one
    token: the widths' single-token kernels on two streams); a width left out
    of the mask (unless it is the shared expert's), and a width-0 (absent)
    expert, leave their slots untouched. The combine done in the same call
    is bit-identical to moe_combine over the y_slots the call leaves (slots
    of other calls read back, zero weights skipped)."""
    H, I, E, k = 256, 128, 9, 4
    made = {b: make_experts(moe, orc, syn, b, H, I, E, seed=70) for b in (8, 4, 2)}
    bits = np.array([8, 4, 2, 4, 2, 8, 4, 0, 2], np.uint8)
    table = made[4][0].table.clone()
    for e in range(E):
        if bits[e] in (8, 2):
            table[e] = made[int(bits[e])][0].table[e]
    x = syn.hidden(71, T, H)
    xq_o, sx_o = orc.quantize_act(x)
    idx = random_routing(syn, T, E, k, 72)
    idx[0, :] = [7, 0, 1, 2]  # the first token also names the absent expert
    wts = np.abs(syn.normal(73, syn.stream_id(syn.K_MISC, 73), (T, k))).astype(np.float32)
    wts[0, 2] = 0.0  # a zero weight: that slot is skipped
    for widths in ((8, 4, 2), (4, 2)):
        log(f"mixed T={T} shared_bits={shared_bits} widths={widths}")
        y = torch.full((T, k + 1, H), 7.0, dtype=torch.float32, device="cuda")
        out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        sh = made[shared_bits][1].struct(0) if shared_bits else None
        moe.moe_expert_ffn_mixed(ctx, table, sh, shared_bits or 0, dev(bits), widths, dev(xq_o), dev(sx_o), dev(idx),
                                 H, I, E, y, topk_w=dev(wts), out=out)
        ctx.check()
        ref = torch.empty_like(out)
        moe.moe_combine(ctx, y, dev(wts), shared_bits is not None, ref)
        assert np.array_equal(host(out).view(np.uint32), host(ref).view(np.uint32)), widths
        yg = host(y)
        for t in range(T):
            for j in range(k):
                e = idx[t, j]
                b = int(bits[e])
                if b in widths or b == shared_bits:  # the shared expert's width is always computed
                    r = orc.expert_token(made[b][2][e], xq_o[t], float(sx_o[t]))
                    assert np.array_equal(yg[t, j].view(np.uint32), r["y"].view(np.uint32)), (widths, t, j)
                else:
                    assert np.all(yg[t, j] == 7.0), (widths, t, j)
            if shared_bits:
                r = orc.expert_token(made[shared_bits][3], xq_o[t], float(sx_o[t]))
                assert np.array_equal(yg[t, k].view(np.uint32), r["y"].view(np.uint32)), (widths, t)
            else:
                assert np.all(yg[t, k] == 7.0)


@pytest.mark.parametrize("H,I", [(512, 192), (256, 64), (6144, 2048)])
@pytest.mark.parametrize("shared_bits", [4, 2, None])
def test_ffn_mixed_one_chain_intermediates(moe, ctx, orc, syn, H, I, shared_bits):
    """One token, int4 and int2 experts in one moe_expert_ffn_mixed call: the
    single chain whose kernels take each slot at its own width (the gate/up
    workgroups split between the widths; the down kernel's lanes each own 32
    elements of every slot, whatever its width). Every captured intermediate
    of every slot bit-exact against the oracle at its expert's width; a slot
    of id -1 and one whose width is absent (0) are left untouched; the combine
    bit-identical to moe_combine."""
    E, k = 8, 6
    log(f"mixed one chain H={H} I={I} shared_bits={shared_bits}")
    made = {b: make_experts(moe, orc, syn, b, H, I, E, seed=140) for b in (4, 2)}
    bits = np.array([4, 2, 2, 4, 0, 2, 4, 4], np.uint8)
    table = made[4][0].table.clone()
    for e in range(E):
        if bits[e] == 2:
            table[e] = made[2][0].table[e]
    xq_o, sx_o = orc.quantize_act(syn.hidden(141, 1, H))
    for rep, ids in enumerate(([[1, 0, 2, 3, 5, 6]], [[6, -1, 4, 1, 3, 2]], [[0, 3, 6, 7, -1, 4]])):
        idx = np.array(ids, np.int32)
        wts = np.abs(syn.normal(142, syn.stream_id(syn.K_MISC, 142, rep), (1, k))).astype(np.float32)
        P = k + 1
        dbg = dict(accg=torch.zeros((P, I), dtype=torch.int32, device="cuda"),
                   accu=torch.zeros((P, I), dtype=torch.int32, device="cuda"),
                   a=torch.zeros((P, I), dtype=torch.float32, device="cuda"),
                   aq=torch.zeros((P, I), dtype=torch.int8, device="cuda"),
                   sa=torch.zeros((P,), dtype=torch.float32, device="cuda"),
                   accd=torch.zeros((P, H), dtype=torch.int32, device="cuda"))
        y = torch.full((1, k + 1, H), 7.0, dtype=torch.float32, device="cuda")
        out = torch.empty((1, H), dtype=torch.float32, device="cuda")
        sh = made[shared_bits][1].struct(0) if shared_bits else None
        ctx.set_debug(dbg)
        try:
            moe.moe_expert_ffn_mixed(ctx, table, sh, shared_bits or 0, dev(bits), (4, 2), dev(xq_o), dev(sx_o),
                                     dev(idx), H, I, E, y, topk_w=dev(wts), out=out)
            ctx.check()
        finally:
            ctx.set_debug(None)
        got = {n: host(t) for n, t in dbg.items()}
        yg = host(y)
        for j in range(k + 1):
            if j == k:
                if not shared_bits:
                    assert np.all(yg[0, k] == 7.0)
                    continue
                ex = made[shared_bits][3]
            else:
                e = int(idx[0, j])
                if e < 0 or bits[e] == 0:
                    assert np.all(yg[0, j] == 7.0), (rep, j)
                    continue
                ex = made[int(bits[e])][2][e]
            r = orc.expert_token(ex, xq_o[0], float(sx_o[0]))
            assert np.array_equal(got["accg"][j], r["accg"]), (rep, j)
            assert np.array_equal(got["accu"][j], r["accu"]), (rep, j)
            assert np.array_equal(got["a"][j].view(np.uint32), r["a"].view(np.uint32)), (rep, j)
            assert np.array_equal(got["aq"][j], r["aq"]), (rep, j)
            assert got["sa"][j] == np.float32(r["sa"]), (rep, j)
            assert np.array_equal(got["accd"][j], r["accd"]), (rep, j)
            assert np.array_equal(yg[0, j].view(np.uint32), r["y"].view(np.uint32)), (rep, j)
        ref = torch.empty_like(out)
        moe.moe_combine(ctx, y, dev(wts), shared_bits is not None, ref)
        assert np.array_equal(host(out).view(np.uint32), host(ref).view(np.uint32)), rep


def test_ffn_mixed_last_width_without_work(moe, ctx, orc, syn):
    """One token, no shared expert, a combine: the width that runs last (int2)
    has none of the token's experts, so its down kernel only combines the
    slots the int4 kernels wrote (no weight row is read)."""
    H, I, E, k = 256, 128, 6, 3
    b4, _, o4, _ = make_experts(moe, orc, syn, 4, H, I, E, seed=75)
    bits = np.array([4, 4, 2, 4, 2, 4], np.uint8)
    xq_o, sx_o = orc.quantize_act(syn.hidden(76, 1, H))
    idx = np.array([[3, 0, 5]], np.int32)
    wts = np.array([[0.5, 0.0, 0.25]], np.float32)
    y = torch.full((1, k + 1, H), 7.0, dtype=torch.float32, device="cuda")
    out = torch.empty((1, H), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn_mixed(ctx, b4.table, None, 0, dev(bits), (4, 2), dev(xq_o), dev(sx_o), dev(idx), H, I, E, y,
                             topk_w=dev(wts), out=out)
    ctx.check()
    yg = host(y)
    for j in range(k):
        r = orc.expert_token(o4[idx[0, j]], xq_o[0], float(sx_o[0]))
        assert np.array_equal(yg[0, j].view(np.uint32), r["y"].view(np.uint32)), j
    assert np.all(yg[0, k] == 7.0)
    ref = torch.empty_like(out)
    moe.moe_combine(ctx, y, dev(wts), False, ref)
    assert np.array_equal(host(out).view(np.uint32), host(ref).view(np.uint32))


def test_ffn_mixed_one_token_graph_replay(moe, ctx, orc, syn):
    """The one-token mixed call (single-token kernels of each width, the
    combine in the last down kernel) captured in a HIP graph for four tokens:
    every replay, with eager work and synchronisations in between, equals the
    eager results, slot by slot and combined."""
    H, I, E, k = 256, 128, 8, 3
    b4, sh4, _, _ = make_experts(moe, orc, syn, 4, H, I, E, seed=78)
    b2, _, _, _ = make_experts(moe, orc, syn, 2, H, I, E, seed=78)
    bits = np.array([4, 2, 4, 2, 4, 4, 2, 4], np.uint8)
    table = torch.where(torch.from_numpy(bits == 4).cuda()[:, None], b4.table, b2.table).contiguous()
    eb = dev(bits)
    toks = []
    for t in range(4):
        xq_o, sx_o = orc.quantize_act(syn.hidden(79 + t, 1, H))
        idx = random_routing(syn, 1, E, k, 80 + t)
        wts = np.abs(syn.normal(81, syn.stream_id(syn.K_MISC, 81, t), (1, k))).astype(np.float32)
        toks.append((dev(xq_o), dev(sx_o), dev(idx), dev(wts)))
    def run(i, y, out):
        xq, sx, idx, wts = toks[i]
        moe.moe_expert_ffn_mixed(ctx, table, sh4.struct(0), 4, eb, (4, 2), xq, sx, idx, H, I, E, y, topk_w=wts,
                                 out=out)
    eager = []
    for i in range(4):
        y = torch.zeros((1, k + 1, H), dtype=torch.float32, device="cuda")
        out = torch.empty((1, H), dtype=torch.float32, device="cuda")
        run(i, y, out)
        torch.cuda.synchronize()
        eager.append((y, out))
    ys = [torch.zeros((1, k + 1, H), dtype=torch.float32, device="cuda") for _ in range(4)]
    outs = [torch.empty((1, H), dtype=torch.float32, device="cuda") for _ in range(4)]
    cap = torch.cuda.Stream()
    old = ctx.stream
    ctx.set_stream(cap)
    g = torch.cuda.CUDAGraph()
    try:
        with torch.cuda.graph(g, stream=cap):
            for i in range(4):
                run(i, ys[i], outs[i])
    finally:
        ctx.set_stream(old)
    for rep in range(3):
        for y in ys:
            y.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i in range(4):
            assert torch.equal(ys[i], eager[i][0]) and torch.equal(outs[i], eager[i][1]), (rep, i)
        run(rep, torch.zeros((1, k + 1, H), dtype=torch.float32, device="cuda"),
            torch.empty((1, H), dtype=torch.float32, device="cuda"))  # eager work between replays
        torch.cuda.synchronize()
    ctx.check()


# --------------------------------------------------------------------------
# combine and the whole layer
# --------------------------------------------------------------------------

@pytest.mark.parametrize("k", [1, 2, 8, 16])
def test_combine(moe, ctx, orc, syn, k):
    """Against the oracle for k up to the largest the entry points accept,
    with and without the shared slot. A slot of weight 0 (dropped by top-p)
    is not read: NaN there leaves the output bit-identical."""
    T, H = 9, 6144
    y = syn.normal(70 + k, syn.stream_id(syn.K_MISC, 70), (T, k + 1, H))
    w = np.abs(syn.normal(70 + k, syn.stream_id(syn.K_MISC, 71), (T, k)))
    if k >= 2:
        w[1::2, 1] = 0.0  # odd tokens drop slot 1
    for has_shared in (True, False):
        out = torch.empty((T, H), dtype=torch.float32, device="cuda")
        moe.moe_combine(ctx, dev(y), dev(w), has_shared, out)
        ys = y if has_shared else np.ascontiguousarray(y[:, :k])
        ref = orc.combine(ys, w, has_shared)
        assert rel_row_err(host(out), ref).max() < 1e-5
        if k >= 2:
            yn = y.copy()
            yn[1::2, 1] = np.nan
            out_n = torch.empty_like(out)
            moe.moe_combine(ctx, dev(yn), dev(w), has_shared, out_n)
            assert torch.equal(out_n, out)


@pytest.mark.parametrize("bits", [4, 8, 2])
def test_layer_tiny_end_to_end(moe, ctx, orc, syn, bits):
    """Tiny layer: hidden 128, 8 routed experts + 1 shared, top-2, intermediate
    64, 32 tokens, seed 0, through quantize_act -> router -> ffn -> combine."""
    from quantized_moe_expert_sigmoid_amd.layer import MoeLayer
    from synth import workloads as wl
    w = wl.TINY
    L = MoeLayer(ctx, w.H, w.I, w.E, w.k, bits=bits)
    oexp = []
    for e in range(w.E):
        g, u, d = wl.expert_fp32(w, e)
        L.set_expert_fp32(e, g, u, d)
        oexp.append(orc.pack_expert(bits, g, u, d))
    g, u, d = wl.shared_fp32(w)
    L.set_shared_fp32(g, u, d)
    osh = orc.pack_expert(bits, g, u, d)
    wr, bias = wl.router_fp32(w)
    L.set_router(wr, bias)
    x = wl.hidden_fp32(w)
    res = L.forward(dev(x))
    ctx.check()
    ref = orc.layer(x, orc.ExpertTable(oexp), osh, w.k, wr=wr, bias=bias)
    _, _, keys, sig = orc.router(x, wr, bias, w.k, want_keys=True)
    assert np.array_equal(host(res["xq"]), ref["xq"])
    near = compare_router(host(res["idx"]), host(res["w"]), ref["idx"], keys, sig)
    assert near == 0
    assert np.array_equal(host(res["y"]), ref["y_slots"])
    err = rel_row_err(host(res["out"]), ref["out"])
    assert err.max() < 1e-3, err.max()


@pytest.mark.parametrize("bits", [4, 8, 2])
@pytest.mark.parametrize("H,I,E,k,shared", [(128, 64, 8, 2, True), (512, 192, 16, 8, True), (256, 128, 8, 3, False)])
def test_layer_t1_fused_intermediates(moe, ctx, orc, syn, bits, H, I, E, k, shared):
    """One token through moe_layer_forward (router+top-k+quant, gate/up, the
    requantisation fused with down and the combine): every captured
    intermediate bit-exact against the oracle, and the output bit-identical to
    the per-step entry points."""
    from quantized_moe_expert_sigmoid_amd.layer import MoeLayer
    log(f"fused t1 bits={bits} H={H} I={I} E={E} k={k} shared={shared}")
    seed = 80 + bits
    L = MoeLayer(ctx, H, I, E, k, bits=bits, has_shared=shared)
    oexp = []
    for e in range(E):
        g, u, d = syn.expert_weights(seed, 0, e, H, I)
        L.set_expert_fp32(e, g, u, d)
        oexp.append(orc.pack_expert(bits, g, u, d))
    osh = None
    if shared:
        g, u, d = syn.expert_weights(seed, 0, 0, H, I, shared=True)
        L.set_shared_fp32(g, u, d)
        osh = orc.pack_expert(bits, g, u, d)
    wr = syn.router_weights(seed, 0, E, H)
    bias = syn.router_bias(seed, 0, E)
    L.set_router(wr, bias)
    S = k + 1
    for tok in range(3):
        x = syn.hidden(seed, 1, H, batch=tok)
        dbg = dict(accg=torch.zeros((S, I), dtype=torch.int32, device="cuda"),
                   accu=torch.zeros((S, I), dtype=torch.int32, device="cuda"),
                   a=torch.zeros((S, I), dtype=torch.float32, device="cuda"),
                   aq=torch.zeros((S, I), dtype=torch.int8, device="cuda"),
                   sa=torch.zeros((S,), dtype=torch.float32, device="cuda"),
                   accd=torch.zeros((S, H), dtype=torch.int32, device="cuda"))
        ctx.set_debug(dbg)
        try:
            res = L.forward(dev(x))
            ctx.check()
        finally:
            ctx.set_debug(None)
        got = {n: host(t) for n, t in dbg.items()}
        fused = {n: host(t).copy() for n, t in res.items()}
        ref = orc.layer(x, orc.ExpertTable(oexp), osh, k, wr=wr, bias=bias)
        _, _, keys, sig = orc.router(x, wr, bias, k, want_keys=True)
        assert compare_router(fused["idx"], fused["w"], ref["idx"], keys, sig) == 0
        assert np.array_equal(fused["xq"], ref["xq"]) and np.array_equal(fused["sx"], ref["sx"])
        for j in range(k + (1 if shared else 0)):
            ex = osh if j == k else oexp[fused["idx"][0, j]]
            r = orc.expert_token(ex, ref["xq"][0], float(ref["sx"][0]))
            assert np.array_equal(got["accg"][j], r["accg"]), j
            assert np.array_equal(got["accu"][j], r["accu"]), j
            assert np.array_equal(got["a"][j].view(np.uint32), r["a"].view(np.uint32)), j
            assert np.array_equal(got["aq"][j], r["aq"]), j
            assert got["sa"][j] == np.float32(r["sa"]), j
            assert np.array_equal(got["accd"][j], r["accd"]), j
            assert np.array_equal(fused["y"][0, j], r["y"]), j
        assert rel_row_err(fused["out"], ref["out"]).max() < 1e-3
        steps = L.forward_steps(dev(x))
        torch.cuda.synchronize()
        assert np.array_equal(host(steps["out"]), fused["out"])
        assert np.array_equal(host(steps["idx"]), fused["idx"])


def _t1_launches(ctx, fn):
    """Kernel launches per stage of one call of fn (the library's timing)."""
    torch.cuda.synchronize()
    ctx.enable_timing(True)
    try:
        fn()
        torch.cuda.synchronize()
        tm = ctx.read_timing()
    finally:
        ctx.enable_timing(False)
    return {name: n for name, (_, n) in tm.items()}


@pytest.mark.parametrize("I", [2112, 4096])
def test_layer_t1_long_intermediate_int2(moe, ctx, orc, syn, I):
    """Past an intermediate of 2048 the single-token path takes int2 layers
    without a shared expert only; its down launch then requantises two float4
    of each slot's a per thread (the second partly filled at 2112). Every
    intermediate bit-exact, and the call is the single-token one (no bucketing,
    one gate/up and one down launch)."""
    test_layer_t1_fused_intermediates(moe, ctx, orc, syn, 2, 256, I, 8, 2, False)
    from quantized_moe_expert_sigmoid_amd.layer import MoeLayer
    L = MoeLayer(ctx, 256, I, 8, 2, bits=2, has_shared=False)
    for e in range(8):
        L.set_expert_fp32(e, *syn.expert_weights(7, 0, e, 256, I))
    L.set_router(syn.router_weights(7, 0, 8, 256), syn.router_bias(7, 0, 8))
    x = dev(syn.hidden(7, 1, 256))
    n = _t1_launches(ctx, lambda: L.forward(x))
    assert n["bucket"] == 0 and n["gateup"] == 1 and n["down"] == 1 and n["requant"] == 0, n


@pytest.mark.parametrize("I", [2112, 4096])
def test_ffn_one_token_long_intermediate_int2(moe, ctx, orc, syn, I):
    """The per-step FFN of one token (routing given) on the single-token
    kernels past an intermediate of 2048 (int2, no shared expert): every
    intermediate bit-exact, with and without dropped slots."""
    test_ffn_one_token(moe, ctx, orc, syn, 2, 256, I, 8, 2, False)
    blocks, _, _, _ = make_experts(moe, orc, syn, 2, 256, I, 8, seed=97)
    xq_o, sx_o = orc.quantize_act(syn.hidden(98, 1, 256))
    y = torch.zeros((1, 3, 256), dtype=torch.float32, device="cuda")
    idx = dev(np.array([[1, 6]], np.int32))
    n = _t1_launches(ctx, lambda: moe.moe_expert_ffn_q2(ctx, blocks.table, None, None, dev(xq_o), dev(sx_o), idx,
                                                         256, I, 8, y))
    assert n["bucket"] == 0 and n["gateup"] == 1 and n["down"] == 1 and n["requant"] == 0, n
