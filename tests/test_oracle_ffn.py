"""Pins of the oracle's fp32 exp/SiLU, expert FFN (O5/O6), combine (O7) and
full layer.

Pages: agentlenshq.com "Colibri ...", section "Key features" (integer-dot
matmuls on int8 operands, dequantisation on use with per-row scales) and
section "Memory split" (shared experts always resident); remio.ai "How Colibri
runs GLM-5.2" (the router picks a few feed-forward modules per token).

Pins: exp against math.exp within a few ulp and at exact points; SiLU
identities; int32 accumulators against numpy integer matmuls over an
independent numpy unpack; the dequantised fp64 brute force; the E = 1, k = 1
layer reducing to one dense SwiGLU FFN against an unquantised fp64 SwiGLU
within the quantisation error; combine against an fp64 numpy sum; identical
experts collapsing the combine.
"""
import math

import numpy as np
import pytest

from tests.test_oracle_quant import numpy_unpack


def test_exp_accuracy(orc):
    xs = np.concatenate([np.linspace(-87, 88, 20001), np.linspace(-1, 1, 2001)]).astype(np.float32)
    worst = 0.0
    for x in xs:
        got = orc.exp_f32(float(x))
        ref = math.exp(float(x))
        worst = max(worst, abs(got - ref) / ref)
    assert worst < 4 * 2.0 ** -24, worst  # within a few fp32 ulp
    assert orc.exp_f32(0.0) == 1.0
    for n in (-20, -1, 1, 10, 100):  # reduction boundaries x = n ln2 (rounded to fp32)
        x = float(np.float32(n * math.log(2)))
        assert orc.exp_f32(x) == pytest.approx(math.exp(x), rel=3e-7)
    assert orc.exp_f32(100.0) == math.inf and orc.exp_f32(-200.0) == 0.0


def test_silu_identities(orc):
    for x in (-9.5, -2.25, -0.3, 0.0, 0.7, 3.0, 12.0):
        s = orc.silu_f32(x)
        ref = x / (1 + math.exp(-x))
        assert s == pytest.approx(ref, rel=1e-6, abs=1e-30)
        # silu(x) - silu(-x) = x
        assert orc.silu_f32(x) - orc.silu_f32(-x) == pytest.approx(x, rel=1e-6, abs=1e-6)
    assert orc.silu_f32(0.0) == 0.0


def make_expert(orc, syn, bits, H, I, seed=0, e=0, shared=False):
    wg, wu, wd = syn.expert_weights(seed, 0, e, H, I, shared=shared)
    return orc.pack_expert(bits, wg, wu, wd), (wg, wu, wd)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_expert_token_integer_accumulators(orc, syn, bits):
    H, I = 256, 96  # H != I so a transposed operand cannot pass
    ex, _ = make_expert(orc, syn, bits, H, I, seed=4, e=bits)
    x = syn.hidden(4, 3, H)
    xq, sx = orc.quantize_act(x)
    qg = numpy_unpack(bits, ex.gate, H).astype(np.int64)
    qu = numpy_unpack(bits, ex.up, H).astype(np.int64)
    qd = numpy_unpack(bits, ex.down, I).astype(np.int64)
    for t in range(3):
        r = orc.expert_token(ex, xq[t], float(sx[t]))
        assert np.array_equal(r["accg"], qg @ xq[t].astype(np.int64))
        assert np.array_equal(r["accu"], qu @ xq[t].astype(np.int64))
        assert np.array_equal(r["accd"], qd @ r["aq"].astype(np.int64))
        # dequantised brute force: sum (qw*sw)(qx*sx) == acc*sw*sx up to rounding
        deq_g = (qg * ex.s_gate[:, None].astype(np.float64)) @ (xq[t].astype(np.float64) * float(sx[t]))
        g = r["accg"].astype(np.float64) * ex.s_gate * float(sx[t])
        assert np.allclose(g, deq_g, rtol=1e-6, atol=1e-9)
        # the SwiGLU intermediate, within fp32 rounding of the fp64 formula
        u = r["accu"].astype(np.float64) * ex.s_up * float(sx[t])
        a64 = g / (1 + np.exp(-g)) * u
        assert np.allclose(r["a"], a64, rtol=2e-6, atol=1e-12)
        # requantisation of a: absmax -> +-127, |a - aq*sa| <= sa/2
        assert r["sa"] == np.float32(np.abs(r["a"]).max()) / np.float32(127)
        assert np.abs(r["aq"]).max() == 127
        assert np.all(np.abs(r["a"] - r["aq"].astype(np.float64) * r["sa"]) <= r["sa"] * (0.5 + 1e-5))
        y = r["accd"].astype(np.float64) * ex.s_down * r["sa"]
        assert np.allclose(r["y"], y, rtol=1e-6, atol=0)


@pytest.mark.parametrize("bits,rel_max,corr_min", [(8, 0.04, 0.999), (4, 0.40, 0.90), (2, None, 0.15)])
def test_dense_special_case_vs_unquantised(orc, syn, bits, rel_max, corr_min):
    """E = 1, k = 1, no shared expert: the layer is one dense SwiGLU FFN. Its
    output tracks the unquantised fp64 SwiGLU within the quantisation error:
    measured relative L2 about 2% (int8) and 24% (int4, worst 30%); ternary
    int2 keeps only a correlation of about 0.26. A wrong sign, a dropped term
    or a transposed operand in the oracle drives the correlation to about 0
    or below."""
    H, I = 512, 192
    ex, (wg, wu, wd) = make_expert(orc, syn, bits, H, I, seed=6)
    x = syn.hidden(6, 8, H)
    res = orc.layer(x, orc.ExpertTable([ex]), None, 1, wr=np.zeros((1, H), np.float32))
    for t in range(8):
        ref = orc.swiglu_f64(wg, wu, wd, x[t])
        out = res["out"][t].astype(np.float64)
        if rel_max is not None:
            rel = np.linalg.norm(out - ref) / np.linalg.norm(ref)
            assert rel < rel_max, rel
        assert np.corrcoef(out, ref)[0, 1] > corr_min
        assert np.allclose(res["w"][t], 1.0)


def test_combine_and_identical_experts(orc, syn):
    T, k, H = 5, 3, 64
    y = syn.normal(9, syn.stream_id(syn.K_MISC, 9), (T, k + 1, H))
    w = np.abs(syn.normal(9, syn.stream_id(syn.K_MISC, 10), (T, k)))
    out = orc.combine(y, w, True)
    ref = y[:, k, :].astype(np.float64) + np.einsum("tj,tjh->th", w.astype(np.float64), y[:, :k].astype(np.float64))
    assert np.allclose(out, ref, rtol=1e-6, atol=1e-7)
    out2 = orc.combine(np.ascontiguousarray(y[:, :k]), w, False)
    assert np.allclose(out2, ref - y[:, k], rtol=1e-5, atol=1e-6)
    # identical routed experts: out = (sum w) * y + y_shared = y + y_shared after normalisation
    H, I, E, kk = 128, 64, 8, 2
    ex, _ = make_expert(orc, syn, 4, H, I, seed=7)
    sh, _ = make_expert(orc, syn, 4, H, I, seed=7, shared=True)
    x = syn.hidden(7, 6, H)
    wr = syn.router_weights(7, 0, E, H)
    res = orc.layer(x, orc.ExpertTable([ex] * E), sh, kk, wr=wr)
    xq, sx = orc.quantize_act(x)
    for t in range(6):
        yy = orc.expert_token(ex, xq[t], float(sx[t]))["y"]
        ys = orc.expert_token(sh, xq[t], float(sx[t]))["y"]
        assert np.allclose(res["out"][t], yy.astype(np.float64) + ys, rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("threads", [1, 4])
def test_tiny_layer_composes_stages(orc, syn, threads):
    """The layer equals its stages run one by one (tiny shape: hidden 128,
    8 experts + 1 shared, top-2, intermediate 64, seed 0), on one thread and
    with its (token, slot) pairs spread over four."""
    assert orc.set_threads(threads) == threads
    T, H, E, k, I = 32, 128, 8, 2, 64
    x = syn.hidden(0, T, H)
    wr = syn.router_weights(0, 0, E, H)
    bias = syn.router_bias(0, 0, E)
    exps = [make_expert(orc, syn, 4, H, I, seed=0, e=e)[0] for e in range(E)]
    sh = make_expert(orc, syn, 4, H, I, seed=0, shared=True)[0]
    res = orc.layer(x, orc.ExpertTable(exps), sh, k, wr=wr, bias=bias)
    xq, sx = orc.quantize_act(x)
    idx, w = orc.router(x, wr, bias, k)
    assert np.array_equal(res["xq"], xq) and np.array_equal(res["sx"], sx)
    assert np.array_equal(res["idx"], idx) and np.array_equal(res["w"], w)
    for t in range(T):
        for j in range(k):
            assert np.array_equal(res["y_slots"][t, j], orc.expert_token(exps[idx[t, j]], xq[t], float(sx[t]))["y"])
        assert np.array_equal(res["y_slots"][t, k], orc.expert_token(sh, xq[t], float(sx[t]))["y"])
    assert np.array_equal(res["out"], orc.combine(res["y_slots"], res["w"], True))


def test_missing_expert_raises(orc, syn):
    H, I = 64, 64
    ex, _ = make_expert(orc, syn, 4, H, I)
    x = syn.hidden(0, 2, H)
    z = np.array([[5.0, 0, 0, 0], [0, 0, 0, 5.0]], np.float32)
    with pytest.raises(KeyError):
        orc.layer(x, orc.ExpertTable([ex, ex, ex, None]), None, 1, logits=z)
