"""moe_layer_forward_noalloc, the whole-layer call that allocates nothing
(its scratch is the library's static device array), against
moe_layer_forward on the same inputs, through the C ABI: every output
bit-identical, on consecutive calls whose second is smaller; under HIP graph
capture on a context that never allocated scratch; and a call beyond the
static area's size refused before anything is enqueued.
"""
import numpy as np
import pytest

from tests.gpu_util import log

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

H, I, E, K = 1024, 512, 32, 4


@pytest.fixture(scope="module")
def setup(orc, syn):
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import quantized_moe_expert_sigmoid_amd as moe
    from quantized_moe_expert_sigmoid_amd.layer import MoeLayer
    moe.lib()
    ctx = moe.MoeCtx(0)
    L = MoeLayer(ctx, H, I, E, K, bits=4)
    for e in range(E):
        L.set_expert_fp32(e, *syn.expert_weights(500, 0, e, H, I))
    L.set_shared_fp32(*syn.expert_weights(500, 0, 0, H, I, shared=True))
    L.set_router(syn.router_weights(500, 0, E, H), syn.router_bias(500, 0, E))
    torch.cuda.synchronize()
    yield moe, ctx, L
    ctx.close()


def outputs(T):
    d = "cuda"
    return dict(out=torch.full((T, H), 3.0, device=d), idx=torch.full((T, K), -7, dtype=torch.int32, device=d),
                w=torch.full((T, K), 5.0, device=d), xq=torch.full((T, H), 9, dtype=torch.int8, device=d),
                sx=torch.full((T,), 2.0, device=d), y=torch.full((T, K + 1, H), 7.0, device=d))


def call(moe, fn, ctx, L, x, b):
    fn(ctx, 4, x, L.experts.table, L.shared.struct(0), K, I, b["out"], w_router=L.w_router, bias=L.bias,
       topk_idx=b["idx"], topk_w=b["w"], xq=b["xq"], sx=b["sx"], y_slots=b["y"])


def same(a, b):
    torch.cuda.synchronize()
    for n in a:
        assert torch.equal(a[n].view(torch.int32) if a[n].dtype == torch.float32 else a[n],
                           b[n].view(torch.int32) if b[n].dtype == torch.float32 else b[n]), n


def test_noalloc_equals_layer_forward(setup, syn):
    """Two calls in a row, the second smaller (40 tokens: the multi-token
    path; then one token: the single-token kernels), each bit-identical to
    moe_layer_forward, with and without the optional outputs."""
    moe, ctx, L = setup
    for T in (40, 1):
        log(f"noalloc vs layer_forward, T={T}")
        x = torch.from_numpy(syn.hidden(501, T, H)).cuda()
        ref, got = outputs(T), outputs(T)
        call(moe, moe.moe_layer_forward, ctx, L, x, ref)
        call(moe, moe.moe_layer_forward_noalloc, ctx, L, x, got)
        ctx.check()
        same(ref, got)
        only_out = torch.full((T, H), 3.0, device="cuda")
        moe.moe_layer_forward_noalloc(ctx, 4, x, L.experts.table, L.shared.struct(0), K, I, only_out,
                                      w_router=L.w_router, bias=L.bias)
        ctx.check()
        same({"out": ref["out"]}, {"out": only_out})


def test_noalloc_graph_capture_on_fresh_context(setup, syn):
    """A context that never ran a call (so never allocated scratch) captures
    noalloc calls of 24 and 1 tokens in a HIP graph; every replay, with eager
    work in between, equals moe_layer_forward's results."""
    moe, ctx, L = setup
    xs = [torch.from_numpy(syn.hidden(502, T, H)).cuda() for T in (24, 1)]
    refs = []
    for x in xs:
        b = outputs(x.shape[0])
        call(moe, moe.moe_layer_forward, ctx, L, x, b)
        refs.append(b)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    fresh = moe.MoeCtx(0, stream=cap)
    try:
        bufs = [outputs(x.shape[0]) for x in xs]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for x, b in zip(xs, bufs):
                call(moe, moe.moe_layer_forward_noalloc, fresh, L, x, b)
        for rep in range(3):
            for b in bufs:
                for t in b.values():
                    t.fill_(1)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for b, r in zip(bufs, refs):
                same(r, b)
            extra = outputs(1)
            call(moe, moe.moe_layer_forward_noalloc, ctx, L, xs[1], extra)  # eager work between replays
            torch.cuda.synchronize()
        fresh.check()
    finally:
        fresh.close()


def test_noalloc_refuses_beyond_static_area(setup):
    """A call whose scratch would exceed the static area is MOE_EINVAL, and
    nothing is enqueued (its output keeps its contents)."""
    moe, ctx, L = setup
    Hb, Ib, Eb, Kb, T = 8192, 8192, 8, 4, 200
    x = torch.zeros((T, Hb), device="cuda")
    out = torch.full((T, Hb), 3.0, device="cuda")
    table = torch.zeros((Eb, 6), dtype=torch.int64, device="cuda")
    wr = torch.zeros((Eb, Hb), device="cuda")
    with pytest.raises(moe.MoeError) as ex:
        moe.moe_layer_forward_noalloc(ctx, 4, x, table, None, Kb, Ib, out, w_router=wr)
    assert ex.value.status == moe.MOE_EINVAL and "static area" in str(ex.value)
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    ctx.enable_timing(True)
    try:
        with pytest.raises(moe.MoeError):
            moe.moe_layer_forward_noalloc(ctx, 4, torch.zeros((1, H), device="cuda"), L.experts.table,
                                          L.shared.struct(0), K, I, torch.empty((1, H), device="cuda"),
                                          w_router=L.w_router)
    finally:
        ctx.enable_timing(False)
    ctx.check()
