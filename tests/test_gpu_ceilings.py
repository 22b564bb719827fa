"""The ceiling measurements on the GPU do the work they claim: every
matrix-core instruction ran (exact accumulator sums), and the streaming read
touched every byte (XOR of its outputs equals the buffer's, ragged tails
included). Through the C ABI of libbt_ceilings."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from ternary_weight_decoder_bt_amd import ceilings as cl  # noqa: E402


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


@pytest.mark.parametrize("blocks,iters,a,b", [(1, 1, 1, 1), (7, 33, 3, -2), (512, 1000, -128, 127),
                                              (256, 1 << 20, 1, 1)])
def test_mfma_issue_checksum(dev, blocks, iters, a, b):
    out = torch.full((blocks * 256,), 12345, dtype=torch.int32, device=dev)
    clocks = torch.zeros(4, dtype=torch.int64, device=dev)
    cl.mfma_i8_issue(blocks, iters, a, b, out, clocks)
    torch.cuda.synchronize()
    assert (out == cl.expected_issue_sum(iters, a, b)).all()
    c = clocks.cpu().tolist()
    assert c[2] >= c[0] and c[3] >= c[1]


@pytest.mark.parametrize("nbytes,blocks", [(16, 1), (4096, 3), ((1 << 20) + 48, 64),
                                           (64 << 20, 2048), ((7 << 20) + 16 * 1001, 5)])
def test_stream_read_xor(dev, nbytes, blocks):
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), dtype=torch.int32,
                         generator=g)
    buf = host.to(dev)
    out = torch.full((blocks * 16,), -1, dtype=torch.int32, device=dev)
    cl.stream_read(buf.data_ptr(), nbytes, blocks, out)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32).reshape(-1, 4))
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32).reshape(-1, 4))
    assert np.array_equal(got, want)
    assert cl.wall_clock_khz(0) > 0
