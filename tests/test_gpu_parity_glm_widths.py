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
