"""GPU parity at the GLM-5.2 expert shape (hidden 6144, intermediate 2048,
top-8, one shared expert) for the int8 and int2 widths, which the int4 GLM
tests do not reach: the single-token kernels (T = 1, their int8 and int2
chunk shapes) and the matrix-core path (T = 5).

Shape source: tech.takumi3488.com "Trying colibri", section on the real 744B
model (hidden 6144, top-8); agentlenshq.com "Colibri ...", section "Key
features" (int8, int4 and int2 kernels with per-row scales). Sixteen routed
experts keep the layer small; the per-expert shapes are the full ones.

Checked for every token: packed bytes of every selected expert (bit-exact
against the oracle's own packing), activation codes, router indices (exact
away from near-ties) and weights, every expert output slot (bit-exact) and the
combined output (1e-3 of the row max).
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


@pytest.mark.parametrize("bits", [8, 2])
def test_glm_shape_other_widths(moe, orc, bits):
    from quantized_moe_expert_sigmoid_amd.layer import MoeLayer
    from synth import workloads as wl
    w = wl.Workload("glm_shape_e16", H=6144, I=2048, E=16, k=8, T=5, seed=7)
    ctx = moe.MoeCtx(0)
    try:
        L = MoeLayer(ctx, w.H, w.I, w.E, w.k, bits=bits)
        for e, g, u, d in wl.iter_experts(w, range(w.E)):
            L.set_expert_fp32(e, g, u, d)
        L.set_shared_fp32(*wl.shared_fp32(w))
        wr, bias = wl.router_fp32(w)
        L.set_router(wr, bias)
        torch.cuda.synchronize()
        osh = orc.pack_expert(bits, *wl.shared_fp32(w))
        oexp = {}
        for T in (1, 5):
            log(f"int{bits} GLM shape, T={T}")
            x = wl.hidden_fp32(w, T)
            res = L.forward(torch.from_numpy(x).cuda())
            torch.cuda.synchronize()
            ctx.check()
            got = {k_: v.cpu().numpy() for k_, v in res.items()}
            idx_o, _, keys, sig = orc.router(x, wr, bias, w.k, want_keys=True)
            assert compare_router(got["idx"], got["w"], idx_o, keys, sig) <= 1  # near-ties: any valid choice
            xq_o, sx_o = orc.quantize_act(x)
            assert np.array_equal(got["xq"], xq_o) and np.array_equal(got["sx"], sx_o)
            for t in range(T):
                ys = []
                for j in range(w.k):
                    e = int(got["idx"][t, j])
                    if e not in oexp:
                        oexp[e] = orc.pack_expert(bits, *wl.expert_fp32(w, e))
                        gp, up, dp, sg, su, sd = L.experts.views(e)
                        assert np.array_equal(gp.cpu().numpy(), oexp[e].gate)
                        assert np.array_equal(dp.cpu().numpy(), oexp[e].down)
                        assert np.array_equal(sd.cpu().numpy(), oexp[e].s_down)
                    y = orc.expert_token(oexp[e], xq_o[t], float(sx_o[t]))["y"]
                    assert np.array_equal(got["y"][t, j].view(np.uint32), y.view(np.uint32)), (T, t, j, e)
                    ys.append(y)
                ysh = orc.expert_token(osh, xq_o[t], float(sx_o[t]))["y"]
                assert np.array_equal(got["y"][t, w.k], ysh), (T, t)
                ref = orc.combine(np.stack(ys + [ysh])[None], got["w"][t:t + 1], True)
                err = rel_row_err(got["out"][t:t + 1], ref)
                assert err.max() < 1e-3, err
    finally:
        ctx.close()


def test_glm_shape_mixed_one_token(moe, orc):
    """The pool stack's per-layer call at the GLM expert shape: one token,
    int4 and int2 experts in one moe_expert_ffn_mixed call with the int4
    shared expert and the combine (the single-token kernels with the routing
    given). Every slot bit-exact against the oracle at its expert's width;
    the combined output bit-identical to moe_combine over the same slots and
    within 1e-3 of the row max of the oracle's combine."""
    from quantized_moe_expert_sigmoid_amd.layer import MoeLayer
    from synth import workloads as wl
    w = wl.Workload("glm_shape_e16", H=6144, I=2048, E=16, k=8, T=1, seed=9)
    ctx = moe.MoeCtx(0)
    try:
        L4 = MoeLayer(ctx, w.H, w.I, w.E, w.k, bits=4)
        L2 = MoeLayer(ctx, w.H, w.I, w.E, w.k, bits=2)
        for e, g, u, d in wl.iter_experts(w, range(w.E)):
            (L4 if e % 3 else L2).set_expert_fp32(e, g, u, d)
        L4.set_shared_fp32(*wl.shared_fp32(w))
        torch.cuda.synchronize()
        bits = np.array([4 if e % 3 else 2 for e in range(w.E)], np.uint8)
        table = torch.where(torch.from_numpy(bits == 4).cuda()[:, None], L4.experts.table, L2.experts.table).contiguous()
        osh = orc.pack_expert(4, *wl.shared_fp32(w))
        x = wl.hidden_fp32(w, 1)
        xq_o, sx_o = orc.quantize_act(x)
        rng = np.random.default_rng(11)
        for rep in range(2):
            idx = rng.choice(w.E, size=w.k, replace=False).astype(np.int32)[None, :]
            wts = rng.random((1, w.k)).astype(np.float32)
            log(f"mixed GLM shape, ids {idx[0].tolist()}")
            y = torch.full((1, w.k + 1, w.H), 7.0, dtype=torch.float32, device="cuda")
            out = torch.empty((1, w.H), dtype=torch.float32, device="cuda")
            moe.moe_expert_ffn_mixed(ctx, table, L4.shared.struct(0), 4, torch.from_numpy(bits).cuda(), (4, 2),
                                     torch.from_numpy(xq_o).cuda(), torch.from_numpy(sx_o).cuda(),
                                     torch.from_numpy(idx).cuda(), w.H, w.I, w.E, y,
                                     topk_w=torch.from_numpy(wts).cuda(), out=out)
            ctx.check()
            ref = torch.empty_like(out)
            moe.moe_combine(ctx, y, torch.from_numpy(wts).cuda(), True, ref)
            torch.cuda.synchronize()
            yg, og = y.cpu().numpy(), out.cpu().numpy()
            assert np.array_equal(og.view(np.uint32), ref.cpu().numpy().view(np.uint32))
            ys = []
            for j in range(w.k):
                e = int(idx[0, j])
                ex = orc.pack_expert(int(bits[e]), *wl.expert_fp32(w, e))
                r = orc.expert_token(ex, xq_o[0], float(sx_o[0]))["y"]
                assert np.array_equal(yg[0, j].view(np.uint32), r.view(np.uint32)), (rep, j, e)
                ys.append(r)
            ysh = orc.expert_token(osh, xq_o[0], float(sx_o[0]))["y"]
            assert np.array_equal(yg[0, w.k].view(np.uint32), ysh.view(np.uint32)), rep
            oref = orc.combine(np.stack(ys + [ysh])[None], wts, True)
            assert rel_row_err(og, oref).max() < 1e-3
    finally:
        ctx.close()


def test_glm_shape_mixed_from_fp32(moe, orc):
    """moe_expert_ffn_mixed_x (fp32 hidden states in, the activation rule
    applied inside the call) against moe_quantize_act_i8 followed by
    moe_expert_ffn_mixed, at the GLM expert shape: every slot and the
    combined output bit-identical. Cases: one token with int4 and int2
    experts (the one-chain mixed kernels quantising in gate/up), one token
    whose experts are all int4 (the single-width chain), one token with int8,
    int4 and int2 experts (one chain per width, each quantising), and three
    tokens (the codes made first, then the multi-token path). The int4/int2
    token's slots are also checked against the oracle."""
    from quantized_moe_expert_sigmoid_amd.layer import MoeLayer
    from synth import workloads as wl
    w = wl.Workload("glm_shape_e16", H=6144, I=2048, E=16, k=8, T=3, seed=13)
    ctx = moe.MoeCtx(0)
    try:
        width = np.array([(4, 2, 8)[e % 3] if e < 12 else 4 for e in range(w.E)], np.uint8)
        layers = {b: MoeLayer(ctx, w.H, w.I, w.E, w.k, bits=b) for b in (8, 4, 2)}
        for e, g, u, d in wl.iter_experts(w, range(w.E)):
            layers[int(width[e])].set_expert_fp32(e, g, u, d)
        layers[4].set_shared_fp32(*wl.shared_fp32(w))
        torch.cuda.synchronize()
        sel = torch.from_numpy(width).cuda()[:, None]
        table = torch.where(sel == 8, layers[8].experts.table,
                            torch.where(sel == 4, layers[4].experts.table, layers[2].experts.table)).contiguous()
        bits_d = torch.from_numpy(width).cuda()
        shared = layers[4].shared.struct(0)
        x_all = wl.hidden_fp32(w, 3)
        cases = [
            ("int4 + int2, one token", np.array([[0, 1, 3, 4, 6, 7, 9, 10]], np.int32), 1),
            ("all int4, one token", np.array([[0, 3, 6, 9, 12, 13, 14, 15]], np.int32), 1),
            ("int8 + int4 + int2, one token", np.array([[0, 1, 2, 3, 4, 5, 6, 7]], np.int32), 1),
            ("three tokens", np.array([[0, 1, 3, 4, 6, 7, 9, 10], [2, 5, 8, 11, 12, 13, 14, 15],
                                       [15, 14, 13, 12, 1, 4, 7, 10]], np.int32), 3),
        ]
        rng = np.random.default_rng(17)
        for name, idx, T in cases:
            log(f"fp32-in mixed call: {name}")
            x = torch.from_numpy(np.ascontiguousarray(x_all[:T])).cuda()
            idx_d = torch.from_numpy(idx).cuda()
            wts = torch.from_numpy(rng.random((T, w.k)).astype(np.float32)).cuda()
            mask = 0
            for e in idx.ravel():
                mask |= 1 << int(width[e])
            xq = torch.empty((T, w.H), dtype=torch.int8, device="cuda")
            sx = torch.empty((T,), dtype=torch.float32, device="cuda")
            moe.moe_quantize_act_i8(ctx, x, xq, sx)
            y_q = torch.full((T, w.k + 1, w.H), 7.0, dtype=torch.float32, device="cuda")
            o_q = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
            moe.moe_expert_ffn_mixed(ctx, table, shared, 4, bits_d, mask, xq, sx, idx_d, w.H, w.I, w.E, y_q,
                                     topk_w=wts, out=o_q)
            y_x = torch.full((T, w.k + 1, w.H), 7.0, dtype=torch.float32, device="cuda")
            o_x = torch.empty((T, w.H), dtype=torch.float32, device="cuda")
            moe.moe_expert_ffn_mixed(ctx, table, shared, 4, bits_d, mask, None, None, idx_d, w.H, w.I, w.E, y_x,
                                     topk_w=wts, out=o_x, x=x)
            ctx.check()
            torch.cuda.synchronize()
            assert np.array_equal(y_x.cpu().numpy().view(np.uint32), y_q.cpu().numpy().view(np.uint32)), name
            assert np.array_equal(o_x.cpu().numpy().view(np.uint32), o_q.cpu().numpy().view(np.uint32)), name
            if name.startswith("int4 + int2"):
                xq_o, sx_o = orc.quantize_act(x_all[:1])
                assert np.array_equal(xq.cpu().numpy(), xq_o)
                yg = y_x.cpu().numpy()
                for j in range(w.k):
                    e = int(idx[0, j])
                    ex = orc.pack_expert(int(width[e]), *wl.expert_fp32(w, e))
                    r = orc.expert_token(ex, xq_o[0], float(sx_o[0]))["y"]
                    assert np.array_equal(yg[0, j].view(np.uint32), r.view(np.uint32)), (j, e)
    finally:
        ctx.close()
