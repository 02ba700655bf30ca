"""The streaming-read probe reads every byte of its window: the XOR of the
window's 32-bit words, folded on the host from one dword per workgroup,
equals numpy's over the same bytes, for windows that leave a ragged tail
against the grid, at several grid sizes; bad arguments are refused."""
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


@pytest.mark.parametrize("nbytes,wpc,reps", [(1 << 20, 1, 1), (1_000_016, 4, 3), (3 * 1_048_592, 2, 7), (16, 8, 2)])
def test_probe_reads_every_byte(moe, ctx, nbytes, wpc, reps):
    rng = np.random.default_rng(nbytes % 1000 + wpc)
    host = rng.integers(0, 256, size=4 * nbytes + 48, dtype=np.uint8)
    buf = torch.from_numpy(host).cuda()
    x, us = moe.moe_probe_stream_read(ctx, buf, nbytes, wpc, reps)
    n_windows = buf.numel() // nbytes
    w = (reps - 1) % n_windows
    ref = np.bitwise_xor.reduce(host[w * nbytes:(w + 1) * nbytes].view(np.uint32))
    log(f"probe {nbytes} B wpc {wpc}: {us:.2f} us")
    assert x == int(ref) and us > 0


def test_probe_refusals(moe, ctx):
    buf = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    for args in ((buf, 0, 1, 1), (buf, 24, 1, 1), (buf, 8192, 1, 1), (buf, 4096, 0, 1), (buf, 4096, 65, 1),
                 (buf, 4096, 1, 0)):
        with pytest.raises(moe.MoeError):
            moe.moe_probe_stream_read(ctx, *args)
    with pytest.raises(moe.MoeError):  # misaligned window base
        moe.moe_probe_stream_read(ctx, buf[4:], 1024, 1, 1)
