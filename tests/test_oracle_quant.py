"""Pins of the oracle's quantise/pack (O1) and activation quantisation (O2).

Page: agentlenshq.com "Colibri: running GLM-5.2 744B MoE on consumer
hardware", section "Key features" (packed int4 / int8 / int2 with per-row
scales) and section "Memory split" (about 19 MB per routed int4 expert).

Pins, none of which re-types the oracle's formula:
  * hand-worked golden rows (tests/golden/pack_examples.txt), exact values;
  * exhaustive round trip over every code of every width;
  * an independent numpy bit-level unpack of the packed bytes;
  * elementwise error bound |w - q*s| <= s/2 and absmax -> +-qmax;
  * the GLM-5.2 expert size reproduces the pages' "about 19 MB".
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pack_examples.txt")


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        bits, w, s, q, b = [f.strip() for f in line.split("|")]
        rows.append((int(bits), np.array([float(v) for v in w.split()], np.float32), float(s),
                     np.array([int(v) for v in q.split()], np.int8),
                     np.array([int(v, 16) for v in b.split()], np.uint8)))
    return rows


def numpy_unpack(bits, packed, cols):
    """Independent bit-level unpack (numpy shifts), not the oracle's."""
    packed = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return packed.view(np.int8).reshape(packed.shape[0], cols)
    per = 8 // bits
    fields = [((packed >> (j * bits)) & ((1 << bits) - 1)).astype(np.int16) for j in range(per)]
    u = np.stack(fields, axis=-1).reshape(packed.shape[0], cols)
    return (u - (1 << (bits - 1))).astype(np.int8)


@pytest.mark.parametrize("row", range(4))
def test_golden_rows(orc, row):
    bits, w, s, q, b = _golden_rows()[row]
    packed, scales = orc.quantize_rows(bits, w[None, :])
    assert scales[0] == np.float32(s)
    assert packed[0].tolist() == b.tolist()
    assert orc.unpack_rows(bits, packed, w.size)[0].tolist() == q.tolist()
    assert numpy_unpack(bits, packed, w.size)[0].tolist() == q.tolist()


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_exhaustive_code_roundtrip(orc, bits):
    qmax = orc.QMAX[bits]
    codes = np.arange(-qmax, qmax + 1, dtype=np.int32)
    per = 8 // bits
    n = ((codes.size + per - 1) // per) * per * 4
    rng = np.random.default_rng(1)
    rows = []
    for r in range(16):
        q = rng.choice(codes, size=n)
        q[rng.integers(n)] = qmax * (1 if r % 2 else -1)  # the absmax element
        rows.append(q)
    q = np.array(rows, dtype=np.int32)
    s = np.float32(0.25)  # power of two: q*s is exact and w/s recovers q exactly
    w = (q * s).astype(np.float32)
    packed, scales = orc.quantize_rows(bits, w)
    assert np.all(scales == s)
    assert np.array_equal(orc.unpack_rows(bits, packed, n).astype(np.int32), q)
    assert np.array_equal(numpy_unpack(bits, packed, n).astype(np.int32), q)


@pytest.mark.parametrize("bits", [8, 4, 2])
def test_random_rows_error_bound(orc, syn, bits):
    R, C = 64, 256
    w = syn.normal(3, syn.stream_id(syn.K_MISC, 0, bits), (R, C), 0.02)
    w[5] = 0.0  # a zero row
    packed, s = orc.quantize_rows(bits, w)
    q = numpy_unpack(bits, packed, C).astype(np.float64)
    qmax = orc.QMAX[bits]
    assert s[5] == 0 and np.all(q[5] == 0)
    nz = np.arange(R) != 5
    a = np.abs(w[nz]).max(axis=1).astype(np.float64)
    assert np.allclose(s[nz], a / qmax, rtol=1e-7, atol=0)
    err = np.abs(w[nz].astype(np.float64) - q[nz] * s[nz, None])
    assert np.all(err <= s[nz, None] * (0.5 + 1e-5))
    # the absmax element of every row is coded +-qmax with the sign of w
    am = np.abs(w[nz]).argmax(axis=1)
    rows = np.nonzero(nz)[0]
    assert np.all(q[nz][np.arange(len(am)), am] == np.sign(w[rows, am]) * qmax)
    assert np.all(np.abs(q) <= qmax)


def test_activation_quant(orc, syn):
    x = syn.normal(0, syn.stream_id(syn.K_HIDDEN, 0, 99), (8, 128), 1.0)
    x[3] = 0.0
    xq, sx = orc.quantize_act(x)
    assert sx[3] == 0 and np.all(xq[3] == 0)
    for t in (0, 1, 7):
        assert sx[t] == np.float32(np.abs(x[t]).max()) / np.float32(127)
        err = np.abs(x[t].astype(np.float64) - xq[t].astype(np.float64) * sx[t])
        assert np.all(err <= sx[t] * (0.5 + 1e-5))
        assert np.abs(xq[t]).max() == 127


def test_glm_expert_bytes_match_pages(orc):
    """Three 6144x2048 matrices at int4 plus fp32 row scales = 18,915,328 B:
    the pages' "about 19 MB" per routed expert (agentlenshq "Memory split")."""
    H, I = 6144, 2048
    for bits, want in ((4, 18_915_328), (8, 37_789_696), (2, 9_478_144)):
        b = 2 * I * orc.row_bytes(bits, H) + H * orc.row_bytes(bits, I) + 4 * (2 * I + H)
        assert b == want
    assert abs(18_915_328 / 1e6 - 19) < 0.5
    # 75 sparse layers x top-8 x 18.9 MB ~ the pages' 11 GB of routed weights per token
    assert abs(75 * 8 * 18_915_328 / 1e9 - 11.35) < 0.01
