"""Pins of the oracle's router (O3) and bucketing (O4).

Pages: tech.takumi3488.com "Trying colibri", self-test section (a
DeepSeek-V3-family router); remio.ai "How Colibri runs GLM-5.2" (the router
selects a few experts per token); remio.ai "The RAM wall became a storage
problem" (an expert requested by several batch positions is read once).

Pins: brute force over every k-subset on the tiny shape, a plain sort of the
logits when the bias is zero (sigmoid is monotone), k = E, exact ties, the
normalised weights against scipy's logistic function on numpy logits, and a
brute-force bucket construction.
"""
import itertools

import numpy as np
import pytest
from scipy.special import expit


def tiny_router_inputs(syn, T=32, H=128, E=8, seed=0):
    x = syn.hidden(seed, T, H)
    wr = syn.router_weights(seed, 0, E, H)
    bias = syn.router_bias(seed, 0, E)
    return x, wr, bias


def test_brute_force_subsets(orc, syn):
    x, wr, bias = tiny_router_inputs(syn)
    k = 2
    idx, w, keys, sig = orc.router(x, wr, bias, k, want_keys=True)
    z = x.astype(np.float64) @ wr.astype(np.float64).T
    assert np.allclose(sig, expit(z), rtol=1e-12, atol=0)
    assert np.allclose(keys, expit(z) + bias.astype(np.float64)[None, :], rtol=1e-12, atol=1e-15)
    for t in range(x.shape[0]):
        best = max(itertools.combinations(range(8), k), key=lambda c: (sum(keys[t, list(c)]), [-e for e in c]))
        assert set(idx[t].tolist()) == set(best)
        assert keys[t, idx[t, 0]] >= keys[t, idx[t, 1]]
        # weights from the unbiased sigmoid, normalised (the bias only selects)
        s = expit(z[t, idx[t]])
        assert np.allclose(w[t], s / s.sum(), rtol=1e-6)
        assert abs(float(w[t].sum()) - 1.0) < 1e-6


def test_zero_bias_is_sort_of_logits(orc, syn):
    x, wr, _ = tiny_router_inputs(syn, T=16, H=128, E=64, seed=5)
    k = 8
    idx, w = orc.router(x, wr, None, k)
    z = x.astype(np.float64) @ wr.astype(np.float64).T
    ref = np.argsort(-z, axis=1, kind="stable")[:, :k]
    assert np.array_equal(idx, ref)
    assert np.all(w > 0)


def test_k_equals_E_and_scale(orc, syn):
    x, wr, bias = tiny_router_inputs(syn, T=4)
    idx, w = orc.router(x, wr, bias, 8, routed_scale=2.5)
    assert all(sorted(r) == list(range(8)) for r in idx.tolist())
    assert np.allclose(w.sum(axis=1), 2.5, rtol=1e-6)


def test_exact_ties_lower_index_first(orc):
    z = np.array([[0.5, 1.0, 1.0, -2.0, 1.0, 0.5]], np.float32)
    idx, w = orc.router(z, None, None, 4, logits_in=True)
    assert idx[0].tolist() == [1, 2, 4, 0]
    bias = np.array([0, 0, 0, 0, 0, 1.0], np.float32)
    idx, w = orc.router(z, None, bias, 2, logits_in=True)
    assert idx[0].tolist() == [5, 1]
    s = expit(np.array([0.5, 1.0]))
    assert np.allclose(w[0], s / s.sum(), rtol=1e-6)


def test_logits_in_matches_hidden_path(orc, syn):
    x, wr, bias = tiny_router_inputs(syn, T=8)
    z = (x.astype(np.float64) @ wr.astype(np.float64).T).astype(np.float32)
    i1, w1 = orc.router(x, wr, bias, 2)
    i2, w2 = orc.router(z, None, bias, 2, logits_in=True)
    assert np.array_equal(i1, i2)
    assert np.allclose(w1, w2, rtol=1e-6)


def test_zipf_logits_follow_popularity(orc, syn):
    """Gumbel-top-k on ln p_r + G samples without replacement from p: the most
    popular expert is chosen far more often than the least popular."""
    E, k, T = 256, 8, 2048
    z = syn.zipf_logits(2, 0, T, E, 1.1)
    rank = syn.zipf_rank(2, 0, E)
    idx, _ = orc.router(z, None, None, k, logits_in=True)
    counts = np.bincount(idx.ravel(), minlength=E)
    by_rank = counts[np.argsort(rank)]
    assert by_rank[0] > 0.5 * T  # rank 1 expert is selected by most tokens
    assert by_rank[:8].sum() > by_rank[-128:].sum()


def brute_bucket(idx, E):
    T, k = idx.shape
    lists = [[] for _ in range(E)]
    for t in range(T):
        for j in range(k):
            lists[idx[t, j]].append(t * k + j)
    counts = np.array([len(l) for l in lists], np.int32)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    perm = np.array([i for l in lists for i in l], np.int32)
    return counts, offsets, perm


@pytest.mark.parametrize("T,E,k", [(1, 256, 8), (32, 8, 2), (64, 256, 8), (7, 5, 5)])
def test_bucket_brute_force(orc, syn, T, E, k):
    z = syn.normal(1, syn.stream_id(syn.K_MISC, T, E), (T, E))
    idx, _ = orc.router(z, None, None, k, logits_in=True)
    c, o, p = orc.bucket(idx, E)
    bc, bo, bp = brute_bucket(idx, E)
    assert np.array_equal(c, bc) and np.array_equal(o, bo) and np.array_equal(p, bp)
    assert sorted(p.tolist()) == list(range(T * k))
    assert int(c.sum()) == T * k


def test_bucket_rejects_bad_index(orc):
    with pytest.raises(RuntimeError):
        orc.bucket(np.array([[0, 9]], np.int32), 8)
