"""GPU parity of the matrix-core expert FFN where its K loop stages several
slices of the tokens' codes in LDS, against the oracle, element by element.

The 64-token and one-block tiles stream a row's weight pieces while the
tokens' field-ordered codes pass through LDS in slices of 512 bytes (256 for
the 64-token tiles when experts average 32 or more tokens). The shapes here
make every width's gate/up and down loops run three or more slices with a
partly filled last slice and a last group of lane pieces that is partly past
the row end:

  hidden 1600: int8 rows of 100 pieces (25 steps, 8 or 4 per slice),
               int4 rows of 50 (13 steps), int2 rows of 25 (7 steps);
  intermediate 1088 (down rows: 68 / 34 / 17 pieces) and 576 (36 / 18 / 9).

Per-expert token counts 16, 17, 64, 65 and 129 (one-block and 64-token
tiles, full and with remainders) run in both tiling regimes: 64 experts (few
tokens per expert on average, 512-byte slices, remainders of up to 16 tokens
as one-block tiles) and 6 experts (many per expert: every remainder a
full-size tile, 256-byte slices). The GLM-shape cases (hidden 6144,
intermediate 2048) run the int8 and int2 64-token tiles with top-2 routing
and the shared expert, every slot of every token.

Pages: agentlenshq.com, "Colibri: running GLM-5.2 744B MoE on consumer
hardware", section "Key features" (int8 / int4 / int2 weights with per-row
scales, integer dot products); remio.ai, "Colibri shows how to run GLM-5.2
on a low-spec PC", section "The RAM wall became a storage problem" (an
expert's weights read once for all the batch positions routed to it).
"""
import numpy as np
import pytest

from tests.gpu_util import log

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


def pack_used(moe, ctx, orc, syn, bits, H, I, E, used, seed):
    """Blocks for E experts of which only `used` are packed (the others are
    never read: no token routes to them); the oracle packs the same fp32
    weights itself."""
    blocks = moe.ExpertBlocks(E, bits, H, I)
    shared = moe.ExpertBlocks(1, bits, H, I)
    oexp = {}
    for e in used:
        wg, wu, wd = syn.expert_weights(seed, 0, e, H, I)
        blocks.pack_from_fp32(ctx, e, dev(wg), dev(wu), dev(wd))
        oexp[e] = orc.pack_expert(bits, wg, wu, wd)
    wg, wu, wd = syn.expert_weights(seed, 0, 0, H, I, shared=True)
    shared.pack_from_fp32(ctx, 0, dev(wg), dev(wu), dev(wd))
    osh = orc.pack_expert(bits, wg, wu, wd)
    torch.cuda.synchronize()
    return blocks, shared, oexp, osh


def run_and_compare(moe, ctx, orc, bits, blocks, shared, oexp, osh, xq_o, sx_o, idx, H, I, E, pairs=None):
    """Run the matrix-core FFN with intermediates captured and compare every
    (token, slot) pair listed (all of them by default) with the oracle."""
    T, k = idx.shape
    P = T * (k + 1)
    dbg = dict(accg=torch.zeros((P, I), dtype=torch.int32, device="cuda"),
               accu=torch.zeros((P, I), dtype=torch.int32, device="cuda"),
               a=torch.zeros((P, I), dtype=torch.float32, device="cuda"),
               aq=torch.zeros((P, I), dtype=torch.int8, device="cuda"),
               sa=torch.zeros((P,), dtype=torch.float32, device="cuda"),
               accd=torch.zeros((P, H), dtype=torch.int32, device="cuda"))
    y = torch.full((T, k + 1, H), 7.0, dtype=torch.float32, device="cuda")
    ctx.set_debug(dbg)
    ctx.set_ffn_kernels("mfma")
    try:
        moe.FFN_BY_BITS[bits](ctx, blocks.table, shared.struct(0), None, dev(xq_o), dev(sx_o), dev(idx), H, I, E, y)
        ctx.check()
    finally:
        ctx.set_debug(None)
        ctx.set_ffn_kernels("auto")
    got = {n: host(t) for n, t in dbg.items()}
    yg = host(y)
    if pairs is None:
        pairs = [(t, j) for t in range(T) for j in range(k + 1)]
    for t, j in pairs:
        ex = osh if j == k else oexp[int(idx[t, j])]
        r = orc.expert_token(ex, xq_o[t], float(sx_o[t]))
        p = t * (k + 1) + j
        assert np.array_equal(got["accg"][p], r["accg"]), (t, j)
        assert np.array_equal(got["accu"][p], r["accu"]), (t, j)
        assert np.array_equal(got["a"][p].view(np.uint32), r["a"].view(np.uint32)), (t, j)
        assert np.array_equal(got["aq"][p], r["aq"]), (t, j)
        assert got["sa"][p] == np.float32(r["sa"]), (t, j)
        assert np.array_equal(got["accd"][p], r["accd"]), (t, j)
        assert np.array_equal(yg[t, j].view(np.uint32), r["y"].view(np.uint32)), (t, j)
    return len(pairs)


@pytest.mark.parametrize("H,I", [(1600, 1088), (1600, 576)])
@pytest.mark.parametrize("E", [64, 6])
@pytest.mark.parametrize("bits", [8, 4, 2])
def test_ffn_mfma_multislice(moe, ctx, orc, syn, bits, E, H, I):
    counts = [16, 17, 64, 65, 129]
    ids = np.concatenate([np.full(c, e, np.int32) for e, c in enumerate(counts)])
    rng = np.random.default_rng(1000 + bits)
    idx = rng.permutation(ids).reshape(-1, 1).astype(np.int32)
    T = idx.shape[0]
    regime = "many tokens per expert" if T >= 32 * E else "few tokens per expert"
    log(f"mfma slices bits={bits} H={H} I={I} E={E} T={T} ({regime})")
    blocks, shared, oexp, osh = pack_used(moe, ctx, orc, syn, bits, H, I, E, range(len(counts)), seed=300 + bits)
    x = syn.hidden(310 + bits, T, H)
    xq_o, sx_o = orc.quantize_act(x)
    n = run_and_compare(moe, ctx, orc, bits, blocks, shared, oexp, osh, xq_o, sx_o, idx, H, I, E)
    log(f"  {n} (token, slot) pairs bit-exact")


@pytest.mark.parametrize("T", [130, 40])
@pytest.mark.parametrize("bits", [8, 2])
def test_glm_shape_mfma_tiles(moe, ctx, orc, syn, bits, T):
    """GLM expert shape (hidden 6144, intermediate 2048), 4 experts, top-2
    and the shared expert: T = 130 averages 65 tokens per expert (64-token
    tiles with 256-byte slices, every remainder a full-size tile), T = 40
    averages 20 (512-byte slices). Every slot of every token bit-exact."""
    H, I, E, k = 6144, 2048, 4, 2
    log(f"GLM-shape mfma tiles int{bits} T={T}")
    blocks, shared, oexp, osh = pack_used(moe, ctx, orc, syn, bits, H, I, E, range(E), seed=320 + bits)
    z = syn.normal(330 + bits, syn.stream_id(syn.K_MISC, 330, T), (T, E))
    idx = np.argsort(-z, axis=1, kind="stable")[:, :k].astype(np.int32)
    log(f"  tokens per expert {np.bincount(idx.ravel(), minlength=E).tolist()}")
    x = syn.hidden(340 + bits, T, H)
    xq_o, sx_o = orc.quantize_act(x)
    n = run_and_compare(moe, ctx, orc, bits, blocks, shared, oexp, osh, xq_o, sx_o, idx, H, I, E)
    log(f"  {n} (token, slot) pairs bit-exact")
