"""GPU parity at the full GLM-5.2 layer shape (hidden 6144, 256 routed experts
+ 1 shared, top-8, intermediate 2048, int4), in the launch configuration the
benchmark times, on sampled tokens the oracle computes one by one.

Shape source: tech.takumi3488.com "Trying colibri", section on the real 744B
model (hidden 6144, 256 experts/layer, top-8); agentlenshq.com "Colibri ...",
section "Memory split" (about 19 MB per int4 expert -> intermediate 2048).

One layer's weights (seed 1) serve every batch size below; the batches differ
in their hidden states and, for the Zipf cases, in the given router logits.
Checked per sampled token: packed bytes of every routed expert and of the
shared expert (bit-exact against the oracle's own packing of the same fp32
weights), activation codes, router indices (exact away from near-ties) and
weights, every expert output slot (bit-exact), the combined output (1e-3 of
the row max). Over all tokens: routing validity.
"""
import numpy as np
import pytest

from tests.gpu_util import compare_router, log, rel_row_err

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def glm():
    assert torch.cuda.is_available()
    import bench
    import quantized_moe_expert_sigmoid_amd as moe
    from synth import workloads as wl
    moe.lib()
    ctx = moe.MoeCtx(0)
    log("building GLM layer (257 experts)")
    L = bench.build_gpu_layer(ctx, wl.DECODE1, 4)
    log("built")
    yield moe, ctx, L
    ctx.close()


class OracleExperts:
    """Oracle-side packing of the same fp32 weights, built lazily per expert."""

    def __init__(self, orc, w):
        self.orc, self.w, self.cache = orc, w, {}
        from synth import workloads as wl
        self.wl = wl
        self.shared = orc.pack_expert(4, *wl.shared_fp32(w))

    def get(self, e):
        if e not in self.cache:
            self.cache[e] = self.orc.pack_expert(4, *self.wl.expert_fp32(self.w, e))
        return self.cache[e]


@pytest.fixture(scope="module")
def oexp(orc):
    from synth import workloads as wl
    return OracleExperts(orc, wl.DECODE1)


def check_packed(L, e, ex):
    g, u, d, sg, su, sd = L.experts.views(e) if e >= 0 else L.shared.views(0)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), ex.gate) and np.array_equal(u.cpu().numpy(), ex.up)
    assert np.array_equal(d.cpu().numpy(), ex.down)
    assert np.array_equal(sg.cpu().numpy(), ex.s_gate) and np.array_equal(su.cpu().numpy(), ex.s_up)
    assert np.array_equal(sd.cpu().numpy(), ex.s_down)


def run_and_check(glm, orc, oexp, x, logits, sample, checked_packed):
    moe, ctx, L = glm
    wl = oexp.wl
    w = oexp.w
    T = x.shape[0]
    res = L.forward(torch.from_numpy(x).cuda(), None if logits is None else torch.from_numpy(logits).cuda())
    ctx.check()
    torch.cuda.synchronize()
    got = {k: v.cpu().numpy() for k, v in res.items()}
    wr, bias = wl.router_fp32(w)
    if logits is None:
        idx_o, w_o, keys, sig = orc.router(x, wr, bias, w.k, want_keys=True)
    else:
        idx_o, w_o, keys, sig = orc.router(logits, None, None, w.k, logits_in=True, want_keys=True)
    near = compare_router(got["idx"], got["w"], idx_o, keys, sig)
    assert near <= max(1, T // 100), near
    xq_o, sx_o = orc.quantize_act(x)
    assert np.array_equal(got["xq"], xq_o) and np.array_equal(got["sx"], sx_o)
    if -1 not in checked_packed:
        check_packed(L, -1, oexp.shared)
        checked_packed.add(-1)
    for t in sample:
        ys = []
        for j in range(w.k):
            e = int(got["idx"][t, j])
            ex = oexp.get(e)
            if e not in checked_packed:
                check_packed(L, e, ex)
                checked_packed.add(e)
            y = orc.expert_token(ex, xq_o[t], float(sx_o[t]))["y"]
            assert np.array_equal(got["y"][t, j].view(np.uint32), y.view(np.uint32)), (t, j, e)
            ys.append(y)
        ysh = orc.expert_token(oexp.shared, xq_o[t], float(sx_o[t]))["y"]
        assert np.array_equal(got["y"][t, w.k], ysh)
        ref = orc.combine(np.stack(ys + [ysh])[None], got["w"][t:t + 1], True)
        err = rel_row_err(got["out"][t:t + 1], ref)
        assert err.max() < 1e-3, err
    return got


@pytest.fixture(scope="module")
def packed_seen():
    return set()


def test_glm_decode_t1(glm, orc, oexp, packed_seen):
    from synth import workloads as wl
    for batch in range(3):
        log(f"decode T=1 batch {batch}")
        x = wl.hidden_fp32(wl.DECODE1, 1, batch=batch)
        run_and_check(glm, orc, oexp, x, None, [0], packed_seen)


def test_glm_decode_t64_zipf(glm, orc, oexp, packed_seen):
    from synth import workloads as wl
    log("decode T=64 zipf")
    x = wl.hidden_fp32(wl.DECODE64, 64)
    z = wl.logits_fp32(wl.DECODE64, 64)
    L = glm[2]
    keep, L.bias = L.bias, None  # Zipf logits route without a selection bias
    try:
        got = run_and_check(glm, orc, oexp, x, z, [0, 37, 63], packed_seen)
    finally:
        L.bias = keep
    assert len(np.unique(got["idx"])) < 200  # Zipf concentrates the routing


def test_glm_mtp_verify_t96(glm, orc, oexp, packed_seen):
    from synth import workloads as wl
    log("mtp verify T=96")
    x = wl.hidden_fp32(wl.MTP96, 96)
    run_and_check(glm, orc, oexp, x, None, [5, 95], packed_seen)


def check_expert_tiles(orc, oexp, got, x, e):
    """Every (token, slot) pair of expert e's first 64-token tile and of its
    last tile (the bucket's stable order: ascending token, then slot), each
    slot output bit-exact against the oracle."""
    xq_o, sx_o = orc.quantize_act(x)
    pairs = np.argwhere(got["idx"] == e)  # row-major: ascending (token, slot)
    n = len(pairs)
    last = n - (n % 64 or 64)
    chosen = list(pairs[:64]) + list(pairs[max(last, 64):])
    for t, j in chosen:
        y = orc.expert_token(oexp.get(int(e)), xq_o[t], float(sx_o[t]))["y"]
        assert np.array_equal(got["y"][t, j].view(np.uint32), y.view(np.uint32)), (e, t, j)
    log(f"expert {e}: {n} tokens, {len(chosen)} of them (first and last tile) bit-exact")


def test_glm_prefill_t2048(glm, orc, oexp, packed_seen):
    from synth import workloads as wl
    log("prefill T=2048")
    x = wl.hidden_fp32(wl.PREFILL2048, 2048)
    got = run_and_check(glm, orc, oexp, x, None, [0, 2047], packed_seen)
    counts = np.bincount(got["idx"].ravel(), minlength=256)
    check_expert_tiles(orc, oexp, got, x, int(np.argmax(counts)))


def test_glm_prefill_t2048_zipf(glm, orc, oexp, packed_seen):
    """Zipf prefill: the most popular expert takes most of the 2048 tokens
    (many 64-token tiles of one expert), the tail experts a few each."""
    from synth import workloads as wl
    log("prefill T=2048 zipf")
    x = wl.hidden_fp32(wl.PREFILL2048_ZIPF, 2048)
    z = wl.logits_fp32(wl.PREFILL2048_ZIPF, 2048)
    L = glm[2]
    keep, L.bias = L.bias, None  # Zipf logits route without a selection bias
    try:
        got = run_and_check(glm, orc, oexp, x, z, [1, 1024, 2046], packed_seen)
    finally:
        L.bias = keep
    counts = np.bincount(got["idx"].ravel(), minlength=256)
    assert counts.max() > 1000 and (counts < 16).sum() > 20  # a heavy head and a long tail


def test_glm_graph_replay_matches_eager(glm):
    """The benchmark replays the hot path as a HIP graph: every replay, with
    eager work and synchronisations in between, equals the eager result."""
    from synth import workloads as wl
    moe, ctx, L = glm
    xs = [torch.from_numpy(wl.hidden_fp32(wl.DECODE1, 1, batch=b)).cuda() for b in range(4)]
    eager = []
    for x in xs:
        r = L.forward(x)
        torch.cuda.synchronize()
        eager.append((r["idx"].clone(), r["y"].clone(), r["out"].clone()))
    cap = torch.cuda.Stream()
    old = ctx.stream
    ctx.set_stream(cap)
    g = torch.cuda.CUDAGraph()
    outs = []
    with torch.cuda.graph(g, stream=cap):
        for x in xs:
            r = L.forward(x)
            outs.append(r["out"].clone())
    ctx.set_stream(old)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for i in range(4):
            assert torch.equal(outs[i], eager[i][2]), (rep, i)
        L.forward(xs[rep])  # eager work between replays
        torch.cuda.synchronize()
    ctx.check()


def test_glm_graph_replay_multi_token(glm):
    """Multi-token calls fork the 64-token tiles onto a side stream and join
    back; captured in a graph, every replay (eager work in between) equals the
    eager result, slot by slot and combined."""
    from synth import workloads as wl
    moe, ctx, L = glm
    xs = [torch.from_numpy(wl.hidden_fp32(wl.DECODE64, 64, batch=b)).cuda() for b in range(2)]
    zs = [torch.from_numpy(wl.logits_fp32(wl.DECODE64, 64, batch=b)).cuda() for b in range(2)]
    eager = []
    for x, z in zip(xs, zs):
        r = L.forward(x, z)
        torch.cuda.synchronize()
        eager.append((r["y"].clone(), r["out"].clone()))
    cap = torch.cuda.Stream()
    old = ctx.stream
    ctx.set_stream(cap)
    g = torch.cuda.CUDAGraph()
    outs = []
    with torch.cuda.graph(g, stream=cap):
        for x, z in zip(xs, zs):
            r = L.forward(x, z)
            outs.append((r["y"].clone(), r["out"].clone()))
    ctx.set_stream(old)
    for rep in range(3):
        g.replay()
        torch.cuda.synchronize()
        for i in range(2):
            assert torch.equal(outs[i][0], eager[i][0]), (rep, i)
            assert torch.equal(outs[i][1], eager[i][1]), (rep, i)
        L.forward(xs[rep % 2], zs[rep % 2])
        torch.cuda.synchronize()
    ctx.check()


def test_glm_decode_t1_topp(glm, orc, oexp):
    """The fused single-token path with top-p 0.7 at the GLM shape: kept ids
    and weights as the oracle's truncation, kept slots bit-exact, dropped slots
    zero, the combined output within 1e-3."""
    from synth import workloads as wl
    from tests.gpu_util import compare_topp
    moe, ctx, L = glm
    w = oexp.w
    wr, bias = wl.router_fp32(w)
    p = 0.7
    L.top_p = p
    try:
        for batch in range(3):
            x = wl.hidden_fp32(wl.DECODE1, 1, batch=batch)
            res = L.forward(torch.from_numpy(x).cuda())
            ctx.check()
            got = {k: v.cpu().numpy() for k, v in res.items()}
            idx_o, _, keys, sig = orc.router(x, wr, bias, w.k, want_keys=True)
            assert compare_topp(got["idx"], got["w"], idx_o, keys, sig, p, orc) == 0
            xq_o, sx_o = orc.quantize_act(x)
            ys, ws = [], []
            for j in range(w.k):
                e = int(got["idx"][0, j])
                if e < 0:
                    assert (got["y"][0, j] == 0).all()
                    continue
                y = orc.expert_token(oexp.get(e), xq_o[0], float(sx_o[0]))["y"]
                assert np.array_equal(got["y"][0, j].view(np.uint32), y.view(np.uint32)), (batch, j, e)
                ys.append(y)
                ws.append(got["w"][0, j])
            m = len(ys)
            log(f"top-p {p}: token {batch} keeps {m} of {w.k}")
            ysh = orc.expert_token(oexp.shared, xq_o[0], float(sx_o[0]))["y"]
            assert np.array_equal(got["y"][0, w.k], ysh)
            ref = orc.combine(np.stack(ys + [ysh])[None], np.array([ws], np.float32), True)
            assert rel_row_err(got["out"], ref).max() < 1e-3
    finally:
        L.top_p = 0.0


def test_glm_graph_replay_after_scratch_growth(glm):
    """A graph captured on a fresh context from one-token calls keeps working
    after an eager 64-token call has grown the context's scratch: the buffer
    the graph addresses is kept (not freed) until the context is destroyed,
    so every replay still equals the eager one-token results."""
    from synth import workloads as wl
    moe, ctx0, L = glm
    fresh = moe.MoeCtx(0)
    L.ctx = fresh
    try:
        xs = [torch.from_numpy(wl.hidden_fp32(wl.DECODE1, 1, batch=b)).cuda() for b in range(3)]
        eager = []
        for x in xs:
            r = L.forward(x)
            torch.cuda.synchronize()
            eager.append((r["y"].clone(), r["out"].clone()))
        cap = torch.cuda.Stream()
        fresh.set_stream(cap)
        g = torch.cuda.CUDAGraph()
        outs = []
        with torch.cuda.graph(g, stream=cap):
            for x in xs:
                r = L.forward(x)
                outs.append((r["y"].clone(), r["out"].clone()))
        fresh.set_stream(torch.cuda.current_stream())
        x64 = torch.from_numpy(wl.hidden_fp32(wl.DECODE64, 64)).cuda()
        z64 = torch.from_numpy(wl.logits_fp32(wl.DECODE64, 64)).cuda()
        keep, L.bias = L.bias, None
        try:
            for rep in range(3):
                L.forward(x64, z64)  # grows the scratch on the first pass
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                for i in range(len(xs)):
                    assert torch.equal(outs[i][0], eager[i][0]), (rep, i)
                    assert torch.equal(outs[i][1], eager[i][1]), (rep, i)
        finally:
            L.bias = keep
        fresh.check()
    finally:
        L.ctx = ctx0
        fresh.close()
