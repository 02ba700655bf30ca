"""Pins of the oracle's top-p truncation (orc_topp).

Pages: agentlenshq.com "Colibri: running GLM-5.2 744B MoE on consumer
hardware", measured-benchmark table (the --topp 0.7 setting) and the community
remark that --topp 0.7 alone sped generation up 1.6x (fewer experts loaded per
token). The pages give the option's name and value only; the reading tested
here: in rank order the normalised weights accumulate, the shortest prefix
reaching p is kept and renormalised, the rest are dropped (id -1, weight 0),
p <= 0 disables it.

Pins: a hand-worked case whose sigmoids are exact fractions, the special cases
that reduce to known results (p tiny keeps only the first expert with the full
routed scale; p above 1 or p = 0 reproduces the plain top-k), and invariants
(kept count monotone in p, kept weights summing to the routed scale, kept
weight ratios equal to the plain top-k ratios).
"""
import numpy as np
import pytest


def hand_case():
    # sigmoid(ln 3) = 3/4, sigmoid(0) = 1/2, sigmoid(-ln 3) = 1/4; a fourth
    # expert far below. Top-3 = experts 0, 1, 2 with normalised weights
    # 1/2, 1/3, 1/6 and cumulative weights 1/2, 5/6, 1.
    z = np.array([[np.log(3.0), 0.0, -np.log(3.0), -20.0]], np.float32)
    return z


@pytest.mark.parametrize("p,keep,weights", [
    (0.7, 2, [0.6, 0.4]),        # 1/2 < 0.7 <= 5/6: experts 0 and 1, 3/4 : 1/2 renormalised
    (0.5, 1, [1.0]),             # the first cumulative weight already reaches 1/2
    (0.9, 3, [0.5, 1 / 3, 1 / 6]),
])
def test_hand_worked(orc, p, keep, weights):
    z = hand_case()
    idx, w, _, sig = orc.router(z, None, None, 3, logits_in=True, want_keys=True)
    assert idx[0].tolist() == [0, 1, 2]
    ti, tw, cum = orc.topp(idx, sig, p)
    assert np.allclose(cum[0], [0.5, 5 / 6, 1.0], rtol=1e-6)
    assert ti[0, :keep].tolist() == [0, 1, 2][:keep]
    assert (ti[0, keep:] == -1).all() and (tw[0, keep:] == 0).all()
    assert np.allclose(tw[0, :keep], weights, rtol=1e-6)


def router_case(orc, syn, T=40, E=64, k=8, seed=3):
    z = syn.normal(seed, syn.stream_id(syn.K_MISC, 90, T), (T, E)) * 1.5
    idx, w, _, sig = orc.router(z.astype(np.float32), None, None, k, logits_in=True, want_keys=True)
    return idx, w, sig


def test_special_cases(orc, syn):
    idx, w, sig = router_case(orc, syn)
    # p = 0 and p > 1: the plain top-k, bit for bit
    for p in (0.0, 1.5):
        ti, tw, _ = orc.topp(idx, sig, p, routed_scale=2.5)
        assert np.array_equal(ti, idx)
        if p > 0:  # p = 0 leaves the weights untouched (here zeros from the call)
            assert np.allclose(tw, w * 2.5, rtol=1e-6)
    # p tiny: only the first-ranked expert, carrying the whole routed scale
    ti, tw, _ = orc.topp(idx, sig, 1e-9, routed_scale=2.5)
    assert np.array_equal(ti[:, 0], idx[:, 0]) and (ti[:, 1:] == -1).all()
    assert np.all(tw[:, 0] == np.float32(2.5)) and (tw[:, 1:] == 0).all()


def test_invariants(orc, syn):
    idx, w, sig = router_case(orc, syn)
    prev = None
    for p in np.linspace(0.05, 1.0, 20):
        ti, tw, cum = orc.topp(idx, sig, float(p))
        kept = (ti >= 0).sum(axis=1)
        assert (kept >= 1).all()
        if prev is not None:
            assert (kept >= prev).all()  # a larger p never keeps fewer experts
        prev = kept
        for t in range(idx.shape[0]):
            m = kept[t]
            assert np.array_equal(ti[t, :m], idx[t, :m])  # a rank-order prefix
            assert abs(float(tw[t, :m].sum()) - 1.0) < 1e-6
            assert np.allclose(tw[t, :m] / tw[t, 0], w[t, :m] / w[t, 0], rtol=1e-6)  # ratios of the plain top-k
            # shortest: the prefix before the last kept one stays below p
            if m > 1:
                assert cum[t, m - 2] < p <= cum[t, m - 1] + 1e-15 or m == idx.shape[1]


def test_layer_drops_slots(orc, syn):
    """With top-p, the layer computes only the kept experts: dropped slots are
    zero and the output is the kept slots' weighted sum plus the shared one."""
    from synth import workloads as wl
    w_ = wl.TINY
    oexp = [orc.pack_expert(4, *wl.expert_fp32(w_, e)) for e in range(w_.E)]
    osh = orc.pack_expert(4, *wl.shared_fp32(w_))
    wr, bias = wl.router_fp32(w_)
    x = wl.hidden_fp32(w_)
    full = orc.layer(x, orc.ExpertTable(oexp), osh, w_.k, wr=wr, bias=bias)
    cut = orc.layer(x, orc.ExpertTable(oexp), osh, w_.k, wr=wr, bias=bias, top_p=0.55)
    dropped = cut["idx"] < 0
    assert dropped.any() and (~dropped).any()
    assert np.array_equal(cut["idx"][~dropped], full["idx"][~dropped])
    assert (cut["y_slots"][:, :w_.k][dropped] == 0).all()
    assert np.array_equal(cut["y_slots"][:, :w_.k][~dropped], full["y_slots"][:, :w_.k][~dropped])
    ref = cut["y_slots"][:, w_.k].astype(np.float64) + np.einsum(
        "tk,tkh->th", cut["w"].astype(np.float64), cut["y_slots"][:, :w_.k].astype(np.float64))
    assert np.allclose(cut["out"], ref, rtol=1e-6, atol=1e-6)
